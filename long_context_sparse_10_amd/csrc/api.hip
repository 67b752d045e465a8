// C ABI of libcsa (declared in include/csa.h): host-side argument checks,
// workspace sizing and dispatch to the gfx950 kernels.  Nothing here
// allocates, synchronises or keeps state.
#include <limits.h>

#include "common.hpp"
#include "internal.hpp"

using namespace csa;

namespace {

bool is_f32_bf16(csa_dtype t) { return t == CSA_F32 || t == CSA_BF16; }
bool is_row_fmt(csa_dtype t) {
  return t == CSA_F32 || t == CSA_BF16 || t == CSA_FP8MIX || t == CSA_MXFP4;
}

// checks shared by every producer of stored rows (prep and compress)
csa_status check_row_out(csa_dtype out_t, int c, int rope_dims, float rope_theta, float eps,
                         const void* out, const uint8_t* out_scale) {
  if (!is_row_fmt(out_t)) return CSA_ERR_UNSUPPORTED;
  if (c <= 0 || c > 4096 || (c & 1)) return CSA_ERR_INVALID;
  if (rope_dims < 0 || rope_dims > c || (rope_dims & 1)) return CSA_ERR_INVALID;
  if (rope_dims > 0 && !(rope_theta > 0.f)) return CSA_ERR_INVALID;
  if (!(eps >= 0.f)) return CSA_ERR_INVALID;
  if (out == nullptr) return CSA_ERR_INVALID;
  if (out_t == CSA_FP8MIX && (rope_dims == 0 || rope_dims == c)) return CSA_ERR_INVALID;
  if (out_t == CSA_MXFP4 && (c % 32 != 0 || out_scale == nullptr)) return CSA_ERR_INVALID;
  return CSA_OK;
}

csa_status launch_status(hipError_t e) { return e == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH; }

// workspace protocol: ws_bytes == NULL means the caller offers no workspace
// (fine when none is needed); ws == NULL reports the size; otherwise it must
// be large enough.  Returns true when the call must return *st right away.
bool ws_query(void* ws, size_t* ws_bytes, size_t need, csa_status* st) {
  if (ws_bytes == nullptr) {
    if (need == 0) return false;
    *st = CSA_ERR_WORKSPACE;
    return true;
  }
  if (ws == nullptr) {
    *ws_bytes = need;
    *st = CSA_OK;
    return true;
  }
  if (*ws_bytes < need) {
    *st = CSA_ERR_WORKSPACE;
    return true;
  }
  return false;
}

// host checks of a paged series (rows of rb bytes, at most Nmax entries per
// sequence, bases 16-byte aligned); *pg receives the kernels' view
csa_status check_pages(const csa_pages* p, int Nmax, int64_t rb, const void* base,
                       const void* base2, PageMap* pg) {
  if (p == nullptr || p->block_table == nullptr || p->max_blocks < 1) return CSA_ERR_INVALID;
  if (p->entries_log2 < 0 || p->entries_log2 > 16) return CSA_ERR_INVALID;
  if (p->page_bytes <= 0 || p->page_bytes % 16 != 0) return CSA_ERR_INVALID;
  if ((int64_t)Nmax > ((int64_t)p->max_blocks << p->entries_log2)) return CSA_ERR_INVALID;
  if ((rb << p->entries_log2) > p->page_bytes) return CSA_ERR_INVALID;
  if ((uintptr_t)base % 16 != 0 || (uintptr_t)base2 % 16 != 0) return CSA_ERR_INVALID;
  *pg = PageMap{p->block_table, p->page_bytes, p->max_blocks, p->entries_log2};
  return CSA_OK;
}

}  // namespace

namespace csa {

csa_status check_attend(const AttendArgs& a) {
  if (a.q == nullptr || a.q_pos == nullptr || a.kv == nullptr || a.sink == nullptr ||
      a.out == nullptr)
    return CSA_ERR_INVALID;
  if (a.B < 0 || a.Tq < 0 || a.nh <= 0 || a.c <= 0 || (a.c & 1) || a.Nmax <= 0) return CSA_ERR_INVALID;
  if ((int64_t)a.B * a.Tq * (((a.idx ? a.k : a.Nmax) + a.n_win) / 128 + 1) > (1ll << 31)) return CSA_ERR_INVALID;
  if (a.rope_dims < 0 || a.rope_dims > a.c || (a.rope_dims & 1)) return CSA_ERR_INVALID;
  if (a.rope_dims > 0 && !(a.rope_theta > 0.f)) return CSA_ERR_INVALID;
  if (!(a.eps >= 0.f)) return CSA_ERR_INVALID;
  // slot tables hold int32 row ids
  if (!a.pages.paged() && (int64_t)a.B * a.Nmax > INT_MAX) return CSA_ERR_INVALID;
  if ((int64_t)a.B * a.win_len > INT_MAX - 2) return CSA_ERR_INVALID;
  if (a.n_win < 0 || (a.n_win > 0 && (a.win == nullptr || a.win_len < a.n_win))) return CSA_ERR_INVALID;
  if (!is_f32_bf16(a.q_t) || !is_f32_bf16(a.out_t)) return CSA_ERR_UNSUPPORTED;
  if (!(is_f32_bf16(a.kv_t) || a.kv_t == CSA_FP8MIX)) return CSA_ERR_UNSUPPORTED;
  if (a.kv_t == CSA_FP8MIX && (a.rope_dims == 0 || a.rope_dims == a.c)) return CSA_ERR_INVALID;
  if (a.c > 1024) return CSA_ERR_UNSUPPORTED;
  if (a.idx != nullptr) {
    if (a.k <= 0) return CSA_ERR_INVALID;
  } else {
    if (a.n_entries == nullptr || a.m_prime <= 0) return CSA_ERR_INVALID;
  }
  return CSA_OK;
}

}  // namespace csa

extern "C" {

const char* csa_version(void) { return "libcsa 0.1 (gfx950)"; }

const char* csa_status_string(csa_status s) {
  switch (s) {
    case CSA_OK: return "ok";
    case CSA_ERR_INVALID: return "invalid argument";
    case CSA_ERR_UNSUPPORTED: return "unsupported dtype combination";
    case CSA_ERR_WORKSPACE: return "workspace too small (or over the no-allocation scratch)";
    case CSA_ERR_LAUNCH: return "kernel launch failed";
    default: break;
  }
  return "unknown status";
}

csa_status csa_prep_rows(const void* x, csa_dtype x_t, int64_t rows, int c, const float* norm_w,
                         float eps, int rope_dims, float rope_theta, const int32_t* pos,
                         int rows_per_seq, int pos_stride, int pos_offset, void* out,
                         uint8_t* out_scale, csa_dtype out_t, hipStream_t stream) {
  if (!is_f32_bf16(x_t)) return CSA_ERR_UNSUPPORTED;
  const csa_status st = check_row_out(out_t, c, rope_dims, rope_theta, eps, out, out_scale);
  if (st != CSA_OK) return st;
  if (rows < 0 || rows > (1ll << 24)) return CSA_ERR_INVALID;
  if (x == nullptr) return CSA_ERR_INVALID;
  if (pos == nullptr && rows_per_seq < 1) return CSA_ERR_INVALID;
  if (rows == 0) return CSA_OK;
  return launch_status(launch_prep_rows(x, x_t, rows, c, norm_w, eps, rope_dims, rope_theta, pos,
                                        rows_per_seq < 1 ? 1 : rows_per_seq, pos_stride,
                                        pos_offset, out, out_scale, out_t, stream));
}

}  // extern "C"

static csa_status compress_impl(const void* H, csa_dtype h_t, int B, int T, int d,
                                const void* W_kv_a, const void* W_z_a, const void* W_kv_b,
                                const void* W_z_b, const float* bias_a, const float* bias_b,
                                int m, int overlap, int c, const float* norm_w, float eps,
                                int rope_dims, float rope_theta, int pos_stride, int pos_offset,
                                void* out, uint8_t* out_scale, csa_dtype out_t,
                                const csa_pages* pages, void* ws, size_t* ws_bytes,
                                hipStream_t stream) {
  if (!is_f32_bf16(h_t)) return CSA_ERR_UNSUPPORTED;
  csa_status st = check_row_out(out_t, c, rope_dims, rope_theta, eps, out, out_scale);
  if (st != CSA_OK) return st;
  if (H == nullptr || W_kv_a == nullptr) return CSA_ERR_INVALID;
  if (B <= 0 || T <= 0 || d <= 0 || m <= 0) return CSA_ERR_INVALID;
  if ((int64_t)B * T > INT_MAX || (int64_t)B * (T / m) > (1ll << 24)) return CSA_ERR_INVALID;
  PageMap pg = kDense;
  if (pages != nullptr) {
    st = check_pages(pages, T / m, row_bytes(out_t, c, rope_dims), out,
                     out_t == CSA_MXFP4 ? out_scale : nullptr, &pg);
    if (st != CSA_OK) return st;
  }
  const bool single = (W_z_a == nullptr);
  if (single && (m != 1 || overlap)) return CSA_ERR_INVALID;
  if (!single && bias_a == nullptr) return CSA_ERR_INVALID;
  if (overlap && (W_kv_b == nullptr || W_z_b == nullptr || bias_b == nullptr)) return CSA_ERR_INVALID;
  if (!overlap && (W_kv_b != nullptr || W_z_b != nullptr)) return CSA_ERR_INVALID;
  const int nproj = single ? 1 : (overlap ? 4 : 2);
  const size_t slot = (size_t)B * T * c;
  const int M = B * T;
  // many tokens of bf16: the projections' weights transposed to [c, d] in the
  // workspace, then one grouped launch of the 256 x 256-tile product
  const bool tiled = h_t == CSA_BF16 && d % 64 == 0 && M >= 256 && c >= 16 &&
                     (uintptr_t)H % 16 == 0;
  const size_t p_bytes = (slot * nproj * sizeof(float) + 255) / 256 * 256;
  const size_t wt_bytes = tiled ? (size_t)nproj * c * d * sizeof(uint16_t) : 0;
  if (ws_query(ws, ws_bytes, p_bytes + wt_bytes, &st)) return st;
  float* P = (float*)ws;
  const void* Ws[4] = {W_kv_a, W_z_a, W_kv_b, W_z_b};
  if (tiled) {
    uint16_t* WT = reinterpret_cast<uint16_t*>((char*)ws + p_bytes);
    for (int i = 0; i < nproj; ++i)
      if (launch_transpose_bf16((const uint16_t*)Ws[i], WT + (size_t)i * c * d, d, c, stream) !=
          hipSuccess)
        return CSA_ERR_LAUNCH;
    if (launch_gemm_nt((const uint16_t*)H, d, WT, (int64_t)c * d, P, c, (int64_t)slot, M, c, d,
                       nproj, stream) != hipSuccess)
      return CSA_ERR_LAUNCH;
  } else {
    for (int i = 0; i < nproj; ++i) {
      const hipError_t e = launch_gemm(H, Ws[i], h_t, P + i * slot, M, c, d, stream);
      if (e != hipSuccess) return CSA_ERR_LAUNCH;
    }
  }
  return launch_status(launch_pool(P, single ? nullptr : P + slot, overlap ? P + 2 * slot : nullptr,
                                   overlap ? P + 3 * slot : nullptr, bias_a, bias_b, B, T, m, c,
                                   norm_w, eps, rope_dims, rope_theta, pos_stride, pos_offset,
                                   out, out_scale, out_t, stream, nullptr, T / m, pg));
}

static csa_status compress_append_impl(const void* H, csa_dtype h_t, int B, int d,
                                       const void* W_kv_a, const void* W_z_a,
                                       const void* W_kv_b, const void* W_z_b,
                                       const float* bias_a, const float* bias_b, int m,
                                       int overlap, int c, const float* norm_w, float eps,
                                       int rope_dims, float rope_theta, int pos_stride,
                                       int pos_offset, const int32_t* entry, void* cache,
                                       uint8_t* cache_scale, csa_dtype out_t, int Nmax,
                                       const csa_pages* pages, void* ws, size_t* ws_bytes,
                                       hipStream_t stream) {
  if (!is_f32_bf16(h_t)) return CSA_ERR_UNSUPPORTED;
  csa_status st = check_row_out(out_t, c, rope_dims, rope_theta, eps, cache, cache_scale);
  if (st != CSA_OK) return st;
  if (H == nullptr || W_kv_a == nullptr || W_z_a == nullptr || bias_a == nullptr ||
      entry == nullptr)
    return CSA_ERR_INVALID;
  if (B < 0 || d <= 0 || m <= 0 || Nmax <= 0) return CSA_ERR_INVALID;
  if (overlap && (W_kv_b == nullptr || W_z_b == nullptr || bias_b == nullptr)) return CSA_ERR_INVALID;
  if (!overlap && (W_kv_b != nullptr || W_z_b != nullptr)) return CSA_ERR_INVALID;
  const int T = overlap ? 2 * m : m;  // tail rows per sequence
  if ((int64_t)B * T > INT_MAX || (int64_t)B * Nmax > INT_MAX) return CSA_ERR_INVALID;
  PageMap pg = kDense;
  if (pages != nullptr) {
    st = check_pages(pages, Nmax, row_bytes(out_t, c, rope_dims), cache,
                     out_t == CSA_MXFP4 ? cache_scale : nullptr, &pg);
    if (st != CSA_OK) return st;
  }
  const int nproj = overlap ? 4 : 2;
  const size_t slot = (size_t)B * T * c;
  if (ws_query(ws, ws_bytes, slot * nproj * sizeof(float), &st)) return st;
  if (B == 0) return CSA_OK;
  float* P = (float*)ws;
  const void* Ws[4] = {W_kv_a, W_z_a, W_kv_b, W_z_b};
  for (int i = 0; i < nproj; ++i) {
    const hipError_t e = launch_gemm(H, Ws[i], h_t, P + i * slot, B * T, c, d, stream);
    if (e != hipSuccess) return CSA_ERR_LAUNCH;
  }
  return launch_status(launch_pool(P, P + slot, overlap ? P + 2 * slot : nullptr,
                                   overlap ? P + 3 * slot : nullptr, bias_a, bias_b, B, T, m, c,
                                   norm_w, eps, rope_dims, rope_theta, pos_stride, pos_offset,
                                   cache, cache_scale, out_t, stream, entry, Nmax, pg));
}

static csa_status indexer_impl(const void* qI, const uint8_t* qI_scale, csa_dtype qI_t,
                               const float* w, const void* kI, const uint8_t* kI_scale,
                               csa_dtype kI_t, const csa_pages* pages, const int32_t* q_pos,
                               const int32_t* n_entries, int B, int Tq, int nI, int cI, int Nmax,
                               int m, void* scores, csa_dtype score_t, hipStream_t stream) {
  if (qI == nullptr || w == nullptr || kI == nullptr || q_pos == nullptr ||
      n_entries == nullptr || scores == nullptr)
    return CSA_ERR_INVALID;
  if (B < 0 || Tq < 0 || nI <= 0 || cI <= 0 || Nmax <= 0 || m <= 0) return CSA_ERR_INVALID;
  if ((int64_t)B * Tq * ((Nmax + 255) / 256) > (1ll << 31)) return CSA_ERR_INVALID;
  if (qI_t != kI_t) return CSA_ERR_UNSUPPORTED;
  if (!(qI_t == CSA_F32 || qI_t == CSA_BF16 || qI_t == CSA_MXFP4)) return CSA_ERR_UNSUPPORTED;
  if (!is_f32_bf16(score_t)) return CSA_ERR_UNSUPPORTED;
  if (qI_t == CSA_MXFP4 && (cI % 32 != 0 || qI_scale == nullptr || kI_scale == nullptr))
    return CSA_ERR_INVALID;
  if ((int64_t)nI * cI > 15 * 1024) return CSA_ERR_UNSUPPORTED;
  PageMap pg = kDense;
  if (pages != nullptr) {
    const csa_status st = check_pages(pages, Nmax, row_bytes(kI_t, cI, 0), kI,
                                      qI_t == CSA_MXFP4 ? kI_scale : nullptr, &pg);
    if (st != CSA_OK) return st;
  }
  if (B == 0 || Tq == 0) return CSA_OK;
  return launch_status(launch_indexer(qI, qI_scale, qI_t, w, kI, kI_scale, q_pos, n_entries, B,
                                      Tq, nI, cI, Nmax, m, scores, score_t, stream, pg));
}

extern "C" {

csa_status csa_compress(const void* H, csa_dtype h_t, int B, int T, int d, const void* W_kv_a,
                        const void* W_z_a, const void* W_kv_b, const void* W_z_b,
                        const float* bias_a, const float* bias_b, int m, int overlap, int c,
                        const float* norm_w, float eps, int rope_dims, float rope_theta,
                        int pos_stride, int pos_offset, void* out, uint8_t* out_scale,
                        csa_dtype out_t, void* ws, size_t* ws_bytes, hipStream_t stream) {
  return compress_impl(H, h_t, B, T, d, W_kv_a, W_z_a, W_kv_b, W_z_b, bias_a, bias_b, m, overlap,
                       c, norm_w, eps, rope_dims, rope_theta, pos_stride, pos_offset, out,
                       out_scale, out_t, nullptr, ws, ws_bytes, stream);
}

csa_status csa_compress_paged(const void* H, csa_dtype h_t, int B, int T, int d,
                              const void* W_kv_a, const void* W_z_a, const void* W_kv_b,
                              const void* W_z_b, const float* bias_a, const float* bias_b, int m,
                              int overlap, int c, const float* norm_w, float eps, int rope_dims,
                              float rope_theta, int pos_stride, int pos_offset, void* out,
                              uint8_t* out_scale, csa_dtype out_t, const csa_pages* pages,
                              void* ws, size_t* ws_bytes, hipStream_t stream) {
  if (pages == nullptr) return CSA_ERR_INVALID;
  return compress_impl(H, h_t, B, T, d, W_kv_a, W_z_a, W_kv_b, W_z_b, bias_a, bias_b, m, overlap,
                       c, norm_w, eps, rope_dims, rope_theta, pos_stride, pos_offset, out,
                       out_scale, out_t, pages, ws, ws_bytes, stream);
}

csa_status csa_compress_append(const void* H, csa_dtype h_t, int B, int d, const void* W_kv_a,
                               const void* W_z_a, const void* W_kv_b, const void* W_z_b,
                               const float* bias_a, const float* bias_b, int m, int overlap, int c,
                               const float* norm_w, float eps, int rope_dims, float rope_theta,
                               int pos_stride, int pos_offset, const int32_t* entry,
                               void* cache, uint8_t* cache_scale, csa_dtype out_t, int Nmax,
                               void* ws, size_t* ws_bytes, hipStream_t stream) {
  return compress_append_impl(H, h_t, B, d, W_kv_a, W_z_a, W_kv_b, W_z_b, bias_a, bias_b, m,
                              overlap, c, norm_w, eps, rope_dims, rope_theta, pos_stride,
                              pos_offset, entry, cache, cache_scale, out_t, Nmax, nullptr, ws,
                              ws_bytes, stream);
}

csa_status csa_compress_append_paged(const void* H, csa_dtype h_t, int B, int d,
                                     const void* W_kv_a, const void* W_z_a, const void* W_kv_b,
                                     const void* W_z_b, const float* bias_a, const float* bias_b,
                                     int m, int overlap, int c, const float* norm_w, float eps,
                                     int rope_dims, float rope_theta, int pos_stride,
                                     int pos_offset, const int32_t* entry, void* cache,
                                     uint8_t* cache_scale, csa_dtype out_t, int Nmax,
                                     const csa_pages* pages, void* ws, size_t* ws_bytes,
                                     hipStream_t stream) {
  if (pages == nullptr) return CSA_ERR_INVALID;
  return compress_append_impl(H, h_t, B, d, W_kv_a, W_z_a, W_kv_b, W_z_b, bias_a, bias_b, m,
                              overlap, c, norm_w, eps, rope_dims, rope_theta, pos_stride,
                              pos_offset, entry, cache, cache_scale, out_t, Nmax, pages, ws,
                              ws_bytes, stream);
}

csa_status indexer_score(const void* qI, const uint8_t* qI_scale, csa_dtype qI_t, const float* w,
                         const void* kI, const uint8_t* kI_scale, csa_dtype kI_t,
                         const int32_t* q_pos, const int32_t* n_entries, int B, int Tq, int nI,
                         int cI, int Nmax, int m, void* scores, csa_dtype score_t,
                         hipStream_t stream) {
  return indexer_impl(qI, qI_scale, qI_t, w, kI, kI_scale, kI_t, nullptr, q_pos, n_entries, B, Tq,
                      nI, cI, Nmax, m, scores, score_t, stream);
}

csa_status indexer_score_paged(const void* qI, const uint8_t* qI_scale, csa_dtype qI_t,
                               const float* w, const void* kI, const uint8_t* kI_scale,
                               csa_dtype kI_t, const csa_pages* pages, const int32_t* q_pos,
                               const int32_t* n_entries, int B, int Tq, int nI, int cI, int Nmax,
                               int m, void* scores, csa_dtype score_t, hipStream_t stream) {
  if (pages == nullptr) return CSA_ERR_INVALID;
  return indexer_impl(qI, qI_scale, qI_t, w, kI, kI_scale, kI_t, pages, q_pos, n_entries, B, Tq,
                      nI, cI, Nmax, m, scores, score_t, stream);
}

csa_status topk_select(const void* scores, csa_dtype score_t, const int32_t* q_pos,
                       const int32_t* n_entries, int B, int Tq, int Nmax, int m, int k,
                       int32_t* idx, void* ws, size_t* ws_bytes, hipStream_t stream) {
  if (scores == nullptr || q_pos == nullptr || n_entries == nullptr || idx == nullptr)
    return CSA_ERR_INVALID;
  if (B < 0 || Tq < 0 || Nmax <= 0 || m <= 0 || k <= 0) return CSA_ERR_INVALID;
  if ((int64_t)B * Tq > INT_MAX) return CSA_ERR_INVALID;
  if (!is_f32_bf16(score_t)) return CSA_ERR_UNSUPPORTED;
  csa_status st;
  if (ws_query(ws, ws_bytes, topk_workspace(B, Tq, Nmax), &st)) return st;
  if (B == 0 || Tq == 0) return CSA_OK;
  return launch_status(launch_topk(scores, score_t, q_pos, n_entries, B, Tq, Nmax, m, k, idx, ws,
                                   stream));
}

csa_status grouped_out_proj(const void* o, csa_dtype t, int R, int nh, int c, int g, int d_g,
                            const void* W_a, const void* W_b, int d, void* y, csa_dtype y_t,
                            void* ws, size_t* ws_bytes, hipStream_t stream) {
  if (o == nullptr || W_a == nullptr || W_b == nullptr || y == nullptr) return CSA_ERR_INVALID;
  if (R < 0 || nh <= 0 || c <= 0 || g <= 0 || d_g <= 0 || d <= 0 || nh % g != 0)
    return CSA_ERR_INVALID;
  if (!is_f32_bf16(t) || !is_f32_bf16(y_t)) return CSA_ERR_UNSUPPORTED;
  const int64_t K1 = (int64_t)nh / g * c, Ku = (int64_t)g * d_g;
  if (K1 > INT_MAX || Ku > INT_MAX || (int64_t)R * nh * c > (1ll << 40) || R > (1 << 24))
    return CSA_ERR_INVALID;
  if (t == CSA_BF16) {
    if (K1 % 32 != 0 || Ku % 32 != 0) return CSA_ERR_INVALID;
    if ((uintptr_t)o % 16 || (uintptr_t)W_a % 16 || (uintptr_t)W_b % 16 || (uintptr_t)y % 16 ||
        (uintptr_t)ws % 16)
      return CSA_ERR_INVALID;
  }
  csa_status st;
  if (ws_query(ws, ws_bytes, oproj_workspace(R, nh, c, g, d_g, d, t), &st)) return st;
  if (R == 0) return CSA_OK;
  return launch_status(launch_oproj(o, t, R, nh, c, g, d_g, W_a, W_b, d, y, y_t, ws, stream));
}

static csa_status attend_common(AttendArgs& a, const csa_pages* pages, void* ws,
                                size_t* ws_bytes, hipStream_t stream) {
  a.pages = kDense;
  if (pages != nullptr) {
    const csa_status sp = check_pages(pages, a.Nmax, row_bytes(a.kv_t, a.c, a.rope_dims), a.kv,
                                      nullptr, &a.pages);
    if (sp != CSA_OK) return sp;
  }
  csa_status st = check_attend(a);
  if (st != CSA_OK) return st;
  if (ws_query(ws, ws_bytes, attend_workspace(a), &st)) return st;
  if (a.B == 0 || a.Tq == 0) return CSA_OK;
  return launch_status(launch_attend(a, ws, stream));
}

csa_status sparse_mqa_attend(const void* q, csa_dtype q_t, const float* q_norm_w, float eps,
                             int rope_dims, float rope_theta, const int32_t* q_pos,
                             const void* kv, csa_dtype kv_t, int Nmax, const int32_t* idx, int k,
                             const void* win, int win_len, int n_win, const float* sink,
                             float scale, int B, int Tq, int nh, int c, void* out,
                             csa_dtype out_t, void* ws, size_t* ws_bytes, hipStream_t stream) {
  if (idx == nullptr) return CSA_ERR_INVALID;
  AttendArgs a{q, q_t, q_norm_w, eps, rope_dims, rope_theta, q_pos, kv, kv_t, Nmax, idx, k,
               nullptr, 0, win, win_len, n_win, sink, scale, B, Tq, nh, c, out, out_t, kDense};
  return attend_common(a, nullptr, ws, ws_bytes, stream);
}

csa_status sparse_mqa_attend_paged(const void* q, csa_dtype q_t, const float* q_norm_w, float eps,
                                   int rope_dims, float rope_theta, const int32_t* q_pos,
                                   const void* kv, csa_dtype kv_t, int Nmax,
                                   const csa_pages* pages, const int32_t* idx, int k,
                                   const void* win, int win_len, int n_win, const float* sink,
                                   float scale, int B, int Tq, int nh, int c, void* out,
                                   csa_dtype out_t, void* ws, size_t* ws_bytes,
                                   hipStream_t stream) {
  if (idx == nullptr || pages == nullptr) return CSA_ERR_INVALID;
  AttendArgs a{q, q_t, q_norm_w, eps, rope_dims, rope_theta, q_pos, kv, kv_t, Nmax, idx, k,
               nullptr, 0, win, win_len, n_win, sink, scale, B, Tq, nh, c, out, out_t, kDense};
  return attend_common(a, pages, ws, ws_bytes, stream);
}

csa_status hca_attend(const void* q, csa_dtype q_t, const float* q_norm_w, float eps,
                      int rope_dims, float rope_theta, const int32_t* q_pos, const void* kv,
                      csa_dtype kv_t, int Nmax, const int32_t* n_entries, int m_prime,
                      const void* win, int win_len, int n_win, const float* sink, float scale,
                      int B, int Tq, int nh, int c, void* out, csa_dtype out_t, void* ws,
                      size_t* ws_bytes, hipStream_t stream) {
  AttendArgs a{q, q_t, q_norm_w, eps, rope_dims, rope_theta, q_pos, kv, kv_t, Nmax, nullptr, 0,
               n_entries, m_prime, win, win_len, n_win, sink, scale, B, Tq, nh, c, out, out_t,
               kDense};
  return attend_common(a, nullptr, ws, ws_bytes, stream);
}

csa_status hca_attend_paged(const void* q, csa_dtype q_t, const float* q_norm_w, float eps,
                            int rope_dims, float rope_theta, const int32_t* q_pos, const void* kv,
                            csa_dtype kv_t, int Nmax, const csa_pages* pages,
                            const int32_t* n_entries, int m_prime, const void* win, int win_len,
                            int n_win, const float* sink, float scale, int B, int Tq, int nh,
                            int c, void* out, csa_dtype out_t, void* ws, size_t* ws_bytes,
                            hipStream_t stream) {
  if (pages == nullptr) return CSA_ERR_INVALID;
  AttendArgs a{q, q_t, q_norm_w, eps, rope_dims, rope_theta, q_pos, kv, kv_t, Nmax, nullptr, 0,
               n_entries, m_prime, win, win_len, n_win, sink, scale, B, Tq, nh, c, out, out_t,
               kDense};
  return attend_common(a, pages, ws, ws_bytes, stream);
}

}  // extern "C"
