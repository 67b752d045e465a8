// Core attention of CSA and HCA (Evidence Ledger Eqs 18-19, Eq 27, Sections
// 2.3.2-2.3.3; shuhuayu section 03): shared-KV multi-query attention of all
// query heads over the selected (CSA) or all visible (HCA) compressed entries
// plus the sliding window, in ONE softmax whose denominator also holds the
// per-head sink exp(z'_h); each row serves as K and V, and the output is
// rotated back by -q on its RoPE channels.
//
// Every query row walks a virtual list of slots: [0, kslots) are compressed
// entries (CSA: idx slots, -1 = empty; HCA: entry s, valid while s < N(q)),
// then n_win window slots for positions q-n_win+1 .. q (negative = empty).
//
// Kernels
//  * attend_mfma_kernel   -- c = 512, heads a multiple of 64, bf16 or
//    FP8/BF16 KV.  One 512-thread block per (query row, 64 heads, slot split):
//    four loader waves gather 32-slot tiles of KV rows through a register ring
//    into a double-buffered LDS tile (e4m3 expanded to bf16 on the way); four
//    math waves of 16 heads run S^T = X Q^T and O^T += X^T P^T on
//    v_mfma_f32_16x16x32_bf16 with an fp32 online softmax in registers.
//    With one split the block finishes the output itself; otherwise it writes
//    per-split (m, l) and O / l (bf16) and attend_combine_kernel merges the
//    splits in order.  Used for FP8 rows and for split slot lists (decode):
//    its register ring keeps four tiles in flight per block.
//  * attend_pf_kernel     -- the same math for bf16 rows and bf16 queries when
//    the slot list is not split (prefill, short lists): 256-thread blocks, two
//    per compute unit, each wave loading its own rows straight into shared
//    memory.
//  * attend_generic_kernel -- any shape / fp32: one wave per head, VALU.
#include "common.hpp"
#include "internal.hpp"

namespace csa {

constexpr float kNegBig = -3.0e38f;  // finite "minus infinity" for running maxima
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy2 = 8.0f * kLog2e;  // 8 nats in log2 units

// 2^x by the hardware instruction (relative error ~1 ulp; -inf -> 0)
__device__ __forceinline__ float exp2f_hw(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// acc + the sum of squares of 8 packed bf16 values (v_dot2_f32_bf16 per pair).
// The words are taken as named components: indexing the vector inside an
// unrolled loop made the compiler square word 0 four times.
__device__ __forceinline__ float sumsq_bf16x8(u32x4 w, float acc) {
  const uint32_t w0 = w.x, w1 = w.y, w2 = w.z, w3 = w.w;
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w0), __builtin_bit_cast(bf16x2_t, w0), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w1), __builtin_bit_cast(bf16x2_t, w1), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w2), __builtin_bit_cast(bf16x2_t, w2), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w3), __builtin_bit_cast(bf16x2_t, w3), acc, false);
  return acc;
}
// two fp32 -> packed bf16 (round to nearest even) by v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2_hw(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

struct SlotCtx {
  const uint8_t* kv;
  const uint8_t* win;
  const int32_t* idx_row;  // sparse only
  PageMap pg;              // kv rows: dense or paged
  int64_t win_base;        // b * win_len
  int64_t rb;              // bytes per row
  int b, kslots, nv, qp, n_win, win_len, nmax;
  bool sparse;
  __device__ __forceinline__ const uint8_t* row(int v) const {
    if (v < kslots) {
      int s = v;
      if (sparse) {
        s = idx_row[v];
        if (s < 0 || s >= nmax) return nullptr;   // -1 = empty slot
      } else if (v >= nv) {
        return nullptr;
      }
      return kv + pg.off(b, s, nmax, rb);
    }
    const int pw = qp - n_win + 1 + (v - kslots);
    if (pw < 0 || v - kslots >= n_win) return nullptr;
    return win + (win_base + pw % win_len) * rb;
  }
};

__device__ __forceinline__ SlotCtx make_ctx(const AttendArgs& a, int row) {
  SlotCtx x;
  const int b = row / a.Tq;
  x.kv = (const uint8_t*)a.kv;
  x.win = (const uint8_t*)a.win;
  x.sparse = a.idx != nullptr;
  x.idx_row = x.sparse ? a.idx + (int64_t)row * a.k : nullptr;
  x.pg = a.pages;
  x.b = b;
  x.win_base = (int64_t)b * a.win_len;
  x.rb = row_bytes(a.kv_t, a.c, a.rope_dims);
  x.qp = a.q_pos[row];
  x.kslots = x.sparse ? a.k : a.Nmax;
  x.nmax = a.Nmax;
  x.nv = x.sparse ? 0 : min(min(a.n_entries[b], a.Nmax), (x.qp + 1) / a.m_prime);
  x.n_win = a.n_win;
  x.win_len = a.win_len;
  return x;
}

// ============================================================ generic (VALU)
template <int GEN_MAXI>  // c <= 64 * GEN_MAXI
__global__ __launch_bounds__(256) void attend_generic_kernel(AttendArgs a, Rope rt) {
  extern __shared__ float sq_all[];
  const int row = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int c = a.c, d_r = a.rope_dims;
  float* sq = sq_all + wave * c;
  const SlotCtx ctx = make_ctx(a, row);
  const int nslots = ctx.kslots + a.n_win;
  const int64_t qrb = row_bytes(a.q_t, c, 0);
  for (int h = wave; h < a.nh; h += nw) {
    // query prep: RMSNorm over the head, then RoPE at the query position
    const uint8_t* qrow = (const uint8_t*)a.q + ((int64_t)row * a.nh + h) * qrb;
    float ss = 0.f;
    for (int j = lane; j < c; j += 64) {
      const float v = load_elem(qrow, a.q_t, j);
      sq[j] = v;
      ss += v * v;
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)c + a.eps);
    for (int j = lane; j < c; j += 64) sq[j] = sq[j] * inv * (a.q_norm_w ? a.q_norm_w[j] : 1.f);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    for (int u = lane; u < d_r / 2; u += 64) {
      float cs, sn;
      rope_cs(rt, (double)ctx.qp, u, &cs, &sn);
      const int i0 = c - d_r + 2 * u;
      const float x0 = sq[i0], x1 = sq[i0 + 1];
      sq[i0] = x0 * cs - x1 * sn;
      sq[i0 + 1] = x0 * sn + x1 * cs;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    float qreg[GEN_MAXI], o[GEN_MAXI];
#pragma unroll
    for (int i = 0; i < GEN_MAXI; ++i) {
      const int j = lane + 64 * i;
      qreg[i] = j < c ? sq[j] : 0.f;
      o[i] = 0.f;
    }
    float m_run = kNegBig, l_run = 0.f;
    for (int v = 0; v < nslots; ++v) {
      const uint8_t* xr = ctx.row(v);
      if (xr == nullptr) continue;
      float xv[GEN_MAXI];
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < GEN_MAXI; ++i) {
        const int j = lane + 64 * i;
        xv[i] = j < c ? load_kv_elem(xr, a.kv_t, c, d_r, j) : 0.f;
        dot = fmaf(qreg[i], xv[i], dot);
      }
      const float logit = a.scale * wave_sum(dot);
      const float m_new = fmaxf(m_run, logit);
      const float alpha = expf(m_run - m_new);
      const float p = expf(logit - m_new);
      l_run = l_run * alpha + p;
#pragma unroll
      for (int i = 0; i < GEN_MAXI; ++i) o[i] = fmaf(o[i], alpha, p * xv[i]);
      m_run = m_new;
    }
    const float z = a.sink[h];
    const float M = fmaxf(m_run, z);
    const float f = expf(m_run - M) / (l_run * expf(m_run - M) + expf(z - M));
    uint8_t* orow = (uint8_t*)a.out + ((int64_t)row * a.nh + h) * row_bytes(a.out_t, c, 0);
#pragma unroll
    for (int i = 0; i < GEN_MAXI; ++i) {
      const int j = lane + 64 * i;
      float val = o[i] * f;
      // inverse RoPE: pair (j, j^1) lives in lanes (lane, lane^1)
      const float other = __shfl_xor(val, 1);
      if (j < c && j >= c - d_r) {
        const int u = (j - (c - d_r)) >> 1;
        float cs, sn;
        rope_cs(rt, -(double)ctx.qp, u, &cs, &sn);
        val = (j & 1) ? other * sn + val * cs : val * cs - other * sn;
      }
      if (j < c) {
        if (a.out_t == CSA_F32) reinterpret_cast<float*>(orow)[j] = val;
        else reinterpret_cast<uint16_t*>(orow)[j] = (uint16_t)f32_to_bf16(val);
      }
    }
  }
}

// ============================================================ MFMA (c = 512)
constexpr int AT_C = 512;
constexpr int AT_TILE = 32;
constexpr int AT_LDX = AT_C + 8;  // bf16 per row of the row-major tile (16-byte pad)
constexpr int AT_TAB = 2048;      // slots one block can walk

// Row id of slot v: kv row b*Nmax + s (>= 0), window row -(2 + b*win_len + p % win_len),
// or -1 for an empty slot.
__device__ __forceinline__ int slot_row_id(const SlotCtx& x, int v) {
  if (v < x.kslots) {
    int s = v;
    if (x.sparse) {
      s = x.idx_row[v];
      if (s < 0 || s >= x.nmax) return -1;
    } else if (v >= x.nv) {
      return -1;
    }
    // dense: the row b * Nmax + s; paged: (page << shift) | slot, decoded by kv_addr
    if (x.pg.paged()) return (x.pg.page(x.b, s) << x.pg.shift) | (s & ((1 << x.pg.shift) - 1));
    return (int)((int64_t)x.b * x.nmax + s);
  }
  const int pw = x.qp - x.n_win + 1 + (v - x.kslots);
  if (pw < 0 || v - x.kslots >= x.n_win) return -1;
  return -2 - (int)(x.win_base + pw % x.win_len);
}

// address of the kv row a slot table id (>= 0) names
__device__ __forceinline__ const uint8_t* kv_addr(const SlotCtx& x, int id) {
  if (x.pg.paged())
    return x.kv + (int64_t)(id >> x.pg.shift) * x.pg.page_bytes +
           (int64_t)(id & ((1 << x.pg.shift) - 1)) * x.rb;
  return x.kv + (int64_t)id * x.rb;
}

// Physical LDS row of tile entry e: a bit permutation (e4 -> bit 0, e0 -> 1,
// e1 -> 2, e3 -> 3, e2 -> 4).  With 520-element rows it keeps both access
// patterns below free of conflicts on gfx950's 64 LDS banks: the 16-byte S^T
// operand reads (16 lanes per pass; lane li reads entry 8(li/4) + 4nt + li%4)
// and the 8-byte transpose reads of the P.V operand (32 lanes per pass; lane q
// of group g reads entry 8g + 4h + q/4).
__device__ __forceinline__ int xrow(int e) {
  return ((e >> 4) & 1) | ((e & 1) << 1) | ((e & 2) << 1) | (e & 8) | ((e & 4) << 2);
}

struct AttendSmem {
  uint16_t Q[64][AT_LDX];           // prepared queries of the block's 64 heads (bf16)
  uint16_t X[2][AT_TILE][AT_LDX];   // gathered rows (double-buffered tiles), rows permuted by xrow
  int32_t slot[AT_TAB + 64];
  uint32_t vmask[AT_TAB / 32 + 2];
  float rcs[AT_C / 2][2];           // cos / sin of the query position for each RoPE pair
  f32x4 qc[AT_C / 2];               // query coefficients per channel pair (see attend_mfma_kernel)
  float gq[AT_C];                   // the same outside the RoPE channels: gain x tau x log2 e
};

// load 8 consecutive elements (dims d..d+7) of a q row as fp32
__device__ __forceinline__ void load8(const uint8_t* qrow, csa_dtype t, int d, float* v) {
  if (t == CSA_F32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(qrow + 4 * d);
    const f32x4 a = p[0], b = p[1];
    v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
    v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  } else {
    const u32x4 w = *reinterpret_cast<const u32x4*>(qrow + 2 * d);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// 8 e4m3 codes (two dwords, element order by byte) -> 8 bf16.  The gfx950
// conversion decodes OCP e4m3fn (checked against the format's definition on
// all codes; 0x7F / 0xFF are NaN and never written by the encoders), and an
// e4m3 value has at most 4 significant bits, so keeping the high half of its
// fp32 bits is its exact bf16.
__device__ __forceinline__ u32x4 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  const f32x2 f0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
  const f32x2 f1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
  const f32x2 f2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
  const f32x2 f3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
  auto hi16 = [](f32x2 f) {
    return __builtin_amdgcn_perm(__float_as_uint(f[1]), __float_as_uint(f[0]), 0x07060302u);
  };
  return u32x4{hi16(f0), hi16(f1), hi16(f2), hi16(f3)};
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// 4 bf16 of a tile column: transpose read (gfx950 ds_read_b64_tr_b16).  Within a
// 16-lane group, lane i receives element i%4 of the 8-byte chunks addressed by
// lanes i/4 + 4j (j = 0..3).
__device__ __forceinline__ uint2 tr_read(const uint16_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(uint2, v);
}
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// the same read as two lanes of an operand vector (fills half of a quad in place)
__device__ __forceinline__ u32x2 tr_read2(const uint16_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Final output of one lane's head (single slot split): the sink joins the
// denominator, the row is normalised, and its RoPE channels are rotated back
// by -q (rcs holds cos / sin of the query position per RoPE pair).  The lane
// holds O^T[dim 16nd + 4g + r][head] in log2-unit softmax state (m_run, l_tot).
// `stage` (bf16 output only; may be null): the wave's 16 rows of AT_LDX in
// shared memory, free to overwrite; the rows are then written one 1 KB head
// row per instruction (the same wave reads back what it wrote)
__device__ __forceinline__ void attend_store_out(const AttendArgs& a, int row, int head, int g,
                                                 const f32x4* O, float m_run, float l_tot,
                                                 const float (*rcs)[2], uint16_t* stage = nullptr) {
  const int d_r = a.rope_dims;
  const float z = a.sink[head] * kLog2e;  // sink in log2 units
  const float M = fmaxf(m_run, z);
  const float em = exp2f_hw(m_run - M);
  const float f = em / (l_tot * em + exp2f_hw(z - M));
  uint8_t* orow = (uint8_t*)a.out + ((int64_t)row * a.nh + head) * row_bytes(a.out_t, AT_C, 0);
  const bool staged = stage != nullptr && a.out_t == CSA_BF16;
  const int lane = threadIdx.x & 63, li = lane & 15;
#pragma unroll
  for (int nd = 0; nd < 32; ++nd) {
    const int d0 = 16 * nd + 4 * g;
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = O[nd][r] * f;
    if (16 * nd + 16 > AT_C - d_r) {
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        if (d0 + r >= AT_C - d_r) {
          const float cs = rcs[(d0 + r - (AT_C - d_r)) >> 1][0];
          const float sn = -rcs[(d0 + r - (AT_C - d_r)) >> 1][1];
          const float x0 = v[r], x1 = v[r + 1];
          v[r] = x0 * cs - x1 * sn;
          v[r + 1] = x0 * sn + x1 * cs;
        }
      }
    }
    if (a.out_t == CSA_F32) {
      *reinterpret_cast<f32x4*>(orow + 4 * d0) = f32x4{v[0], v[1], v[2], v[3]};
    } else if (staged) {
      *reinterpret_cast<uint2*>(stage + li * AT_LDX + d0) =
          make_uint2(pack_bf16x2_hw(v[0], v[1]), pack_bf16x2_hw(v[2], v[3]));
    } else {
      *reinterpret_cast<uint2*>(orow + 2 * d0) =
          make_uint2(pack_bf16x2_hw(v[0], v[1]), pack_bf16x2_hw(v[2], v[3]));
    }
  }
  if (staged) {
    // head - li is the wave's first head; its 16 rows are consecutive in out
    uint16_t* o0 = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)row * a.nh + head - li) * AT_C;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      *reinterpret_cast<u32x4*>(o0 + (int64_t)i * AT_C + 8 * lane) =
          *reinterpret_cast<const u32x4*>(stage + i * AT_LDX + 8 * lane);
  }
}

// One 32-slot tile on a math wave of 16 heads (reads X[BUF] of the block's
// shared memory; needs qf, m_run, l_run, O, li, g and the transpose-read
// addresses tr_r0 / tr_r1 / tr_c in scope): S^T, online softmax, O^T.  RAD
// and RQD are how many S^T operand quads and P.V operand quads are read ahead.
#define CSA_TILE(T, BUF, RAD, RQD)                                                            \
{                                                                                             \
  const uint32_t mask = sm.vmask[T];                                                          \
  if (mask != 0u) {                                                                           \
    f32x4 S[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};                      \
    {                                                                                         \
      const uint16_t* xr0 = &sm.X[BUF][xrow(8 * (li >> 2) + (li & 3))][128 * g];              \
      const uint16_t* xr1 = &sm.X[BUF][xrow(8 * (li >> 2) + 4 + (li & 3))][128 * g];          \
      u32x4 ra[RAD], rb4[RAD];                                                                \
      _Pragma("unroll") for (int q = 0; q < (RAD); ++q) {                                     \
        ra[q] = *reinterpret_cast<const u32x4*>(xr0 + 8 * q);                                 \
        rb4[q] = *reinterpret_cast<const u32x4*>(xr1 + 8 * q);                                \
      }                                                                                       \
      _Pragma("unroll") for (int ks = 0; ks < 16; ++ks) {                                     \
        const u32x4 a0 = ra[ks % (RAD)], a1 = rb4[ks % (RAD)];                                \
        if (ks + (RAD) < 16) {                                                                \
          ra[ks % (RAD)] = *reinterpret_cast<const u32x4*>(xr0 + 8 * (ks + (RAD)));           \
          rb4[ks % (RAD)] = *reinterpret_cast<const u32x4*>(xr1 + 8 * (ks + (RAD)));          \
        }                                                                                     \
        S[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a0), qf[ks], S[0], 0, 0, 0); \
        S[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a1), qf[ks], S[1], 0, 0, 0); \
      }                                                                                       \
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (RAD), 1);                              \
      _Pragma("unroll") for (int ks = 0; ks < 16 - (RAD); ++ks) {                             \
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);                                    \
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);                                    \
      }                                                                                       \
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * (RAD), 1);                              \
    }                                                                                         \
    /* logits in log2 units (the queries carry tau * log2 e); masked slots -inf */            \
    float lg[8];                                                                              \
    _Pragma("unroll") for (int nt = 0; nt < 2; ++nt)                                          \
    _Pragma("unroll") for (int r = 0; r < 4; ++r) lg[4 * nt + r] = S[nt][r];                  \
    if (mask != 0xFFFFFFFFu) {                                                                \
      _Pragma("unroll") for (int nt = 0; nt < 2; ++nt)                                        \
      _Pragma("unroll") for (int r = 0; r < 4; ++r)                                           \
        if (!((mask >> (8 * g + 4 * nt + r)) & 1u)) lg[4 * nt + r] = -INFINITY;               \
    }                                                                                         \
    float mx = fmaxf(fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3])),                         \
                     fmaxf(fmaxf(lg[4], lg[5]), fmaxf(lg[6], lg[7])));                        \
    /* lazy rescale: the reference maximum moves only when a logit exceeds it */              \
    /* by more than 8 nats (weights stay below e^8: safe in fp32 sums and bf16 P). */         \
    /* The max across the head's four lane groups is taken only then. */                      \
    if (__any(mx > m_run + kLazy2)) {                                                         \
      mx = fmaxf(mx, __shfl_xor(mx, 16));                                                     \
      mx = fmaxf(mx, __shfl_xor(mx, 32));                                                     \
      const bool grow = mx > m_run + kLazy2;                                                  \
      const float m_new = grow ? mx : m_run;                                                  \
      const float alpha = exp2f_hw(m_run - m_new);                                            \
      l_run *= alpha;                                                                         \
      m_run = m_new;                                                                          \
      _Pragma("unroll") for (int nd = 0; nd < 32; ++nd) O[nd] *= alpha;                       \
    }                                                                                         \
    float pv[8], ps = 0.f;                                                                    \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                           \
      pv[i] = exp2f_hw(lg[i] - m_run);                                                        \
      ps += pv[i];                                                                            \
    }                                                                                         \
    l_run += ps;                                                                              \
    u32x4 pk;                                                                                 \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) pk[i] = pack_bf16x2_hw(pv[2 * i], pv[2 * i + 1]); \
    const bf16x8 pf = __builtin_bit_cast(bf16x8, pk); /* P^T: entries 8g..8g+7 of head li */  \
    {                                                                                         \
      /* O^T += X^T P^T, operands by transpose reads, 8 column blocks ahead */                \
      const uint16_t* c0 = &sm.X[BUF][tr_r0][tr_c];                                           \
      const uint16_t* c1 = &sm.X[BUF][tr_r1][tr_c];                                           \
      /* each pair of 8-byte reads fills the two halves of one operand quad */                \
      u32x4 rq[RQD];                                                                          \
      _Pragma("unroll") for (int q = 0; q < (RQD); ++q) {                                     \
        rq[q].xy = tr_read2(c0 + 16 * q);                                                     \
        rq[q].zw = tr_read2(c1 + 16 * q);                                                     \
      }                                                                                       \
      _Pragma("unroll") for (int nd = 0; nd < 32; ++nd) {                                     \
        O[nd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, rq[nd % (RQD)]), pf, O[nd], 0, 0, 0); \
        if (nd + (RQD) < 32) {                                                                \
          rq[nd % (RQD)].xy = tr_read2(c0 + 16 * (nd + (RQD)));                               \
          rq[nd % (RQD)].zw = tr_read2(c1 + 16 * (nd + (RQD)));                               \
        }                                                                                     \
      }                                                                                       \
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (RQD), 2);                              \
      _Pragma("unroll") for (int nd = 0; nd < 32 - (RQD); ++nd) {                             \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);                                    \
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);                                    \
      }                                                                                       \
      __builtin_amdgcn_sched_group_barrier(0x008, RQD, 2);                                    \
    }                                                                                         \
  }                                                                                           \
}

// One block = one query row x 64 heads x one slot split, 8 waves:
//  * waves 0-3 (math): wave w owns heads 16w..16w+15 and per 32-slot tile runs
//      S^T[e][h] = X[e] . q_h       v_mfma_f32_16x16x32_bf16, A = rows, B = q (LDS)
//      online softmax over e per head (fp32)
//      O^T[d][h] += sum_e X[e][d] P^T[e][h]   A = rows read transposed, B = P^T
//    The rows feeding S^T are permuted (lane li reads entry 8(li/4) + 4nt + li%4)
//    so that each lane's S^T results are exactly the P^T operand it needs
//    (entries 8g..8g+7 of head li): nothing moves between the two contractions.
//  * waves 4-7 (loaders): wave 4+w gathers rows 8w..8w+7 of every tile into
//    registers, up to two tiles ahead of the one being committed, and commits
//    them (expanding e4m3 to bf16) to the LDS tile the math waves are not using.
// One barrier per tile separates the two buffers.
template <int KVF, bool QBF16, int RING>
__global__ __launch_bounds__(512) void attend_mfma_kernel(AttendArgs a, Rope rt, int chunk,
                                                         int nsplit, void* __restrict__ ws) {
  __shared__ __attribute__((aligned(16))) AttendSmem sm;
  const int hgroups = a.nh / 64;
  // Workgroups are dealt to the 8 XCDs round-robin (block i runs on XCD i % 8).
  // All splits and head groups of query row r go to XCD r % 8, so the row's
  // queries and selected KV rows are fetched into one L2 and shared there.
  const int xcd = blockIdx.x & 7, xj = blockIdx.x >> 3;
  const int split = xj % nsplit;
  const int hg = (xj / nsplit) % hgroups;
  const int row = (xj / (nsplit * hgroups)) * 8 + xcd;
  if (row >= a.B * a.Tq) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool math = wave < 4;
  const int mw = wave & 3;  // math: head group of the wave; loader: its rows 8mw..8mw+7
  const int g = lane >> 4, li = lane & 15;
  const int head = 64 * hg + 16 * mw + li;  // the head of this lane's softmax state (math)
  const int d_r = a.rope_dims;
  const float qscale = a.scale * kLog2e;  // queries carry tau * log2 e: logits in log2 units
  const SlotCtx ctx = make_ctx(a, row);
  const int total = ctx.kslots + a.n_win;
  const int v0 = split * chunk;
  const int v1 = min(v0 + chunk, total);
  const int ntiles = v1 > v0 ? (v1 - v0 + AT_TILE - 1) / AT_TILE : 0;
  const int64_t rb = ctx.rb;

  // the query row of a math lane: lane (g, li) takes dims 128g .. 128g+127 of
  // head `head`, the layout of the S^T operand
  const uint8_t* qrow = (const uint8_t*)a.q + ((int64_t)row * a.nh + head) * row_bytes(a.q_t, AT_C, 0);

  // ---- per channel pair p (channels 2p, 2p+1), one per thread: the RoPE
  // angle of the query position (the output's inverse rotation reuses it with
  // the sine negated) and the query coefficients, which fold the RMSNorm gains
  // (g0, g1), the rotation (c, s; 1, 0 outside the RoPE channels) and
  // tau * log2 e into qc = (g0 c, g1 s, g0 s, g1 c) * tau * log2 e: the
  // prepared pair is (inv (qc.x x0 - qc.y x1), inv (qc.z x0 + qc.w x1))
  for (int p = tid; p < AT_C / 2; p += 512) {
    float cs = 1.f, sn = 0.f;
    if (2 * p >= AT_C - d_r) {
      const int u = p - (AT_C - d_r) / 2;
      rope_cs(rt, (double)ctx.qp, u, &cs, &sn);
      sm.rcs[u][0] = cs;
      sm.rcs[u][1] = sn;
    }
    const float g0 = a.q_norm_w != nullptr ? a.q_norm_w[2 * p] : 1.f;
    const float g1 = a.q_norm_w != nullptr ? a.q_norm_w[2 * p + 1] : 1.f;
    sm.qc[p] = f32x4{g0 * cs * qscale, g1 * sn * qscale, g0 * sn * qscale, g1 * cs * qscale};
    // a pair outside the RoPE channels has coefficients (g0 qscale, 0, 0, g1 qscale)
    sm.gq[2 * p] = g0 * 1.f * qscale;
    sm.gq[2 * p + 1] = g1 * 1.f * qscale;
  }
  // ---- slot table and per-tile validity masks (one coalesced pass)
  for (int i = tid; i < ((ntiles * AT_TILE + 63) & ~63); i += 512) {
    const int v = v0 + i;
    const int id = (i < ntiles * AT_TILE && v < v1) ? slot_row_id(ctx, v) : -1;
    sm.slot[i] = id;
    const uint64_t bal = __ballot(id != -1);
    if (lane == 0) {
      sm.vmask[i >> 5] = (uint32_t)bal;
      sm.vmask[(i >> 5) + 1] = (uint32_t)(bal >> 32);
    }
  }
  __syncthreads();  // slot table and RoPE angles ready

  // ---- the math wave's queries (B operand of S^T) to LDS: RMSNorm over the
  // head (its four lane groups), then the coefficient table (gains, RoPE at q,
  // tau * log2 e), bf16.  Each math lane prepares exactly the fragments it
  // later reads back as its operand; kept in shared memory, they can be
  // re-read instead of held through the tile loop.
#define CSA_QPREP()                                                                          \
  if constexpr (QBF16) {                                                                     \
    /* the wave's 16 raw query rows, coalesced: load i takes head 16 mw + i, lane l its */   \
    /* bytes 16 l .. 16 l + 15, into the wave's own rows of sm.Q; the same wave reads */     \
    /* them back in the operand layout (LDS keeps one wave's accesses in order).  The */    \
    /* query dtype is a template parameter so that these loops stay free of branches. */   \
    u32x4 qraw[16];                                                                          \
    const uint8_t* qb = (const uint8_t*)a.q + ((int64_t)row * a.nh + 64 * hg + 16 * mw) * (2 * AT_C); \
    _Pragma("unroll") for (int i = 0; i < 16; ++i)                                           \
      qraw[i] = *reinterpret_cast<const u32x4*>(qb + (int64_t)i * (2 * AT_C) + 16 * lane);     \
    _Pragma("unroll") for (int i = 0; i < 16; ++i)                                           \
      *reinterpret_cast<u32x4*>(&sm.Q[16 * mw + i][8 * lane]) = qraw[i];                    \
    _Pragma("unroll") for (int ks = 0; ks < 16; ++ks)                                        \
      qraw[ks] = *reinterpret_cast<const u32x4*>(&sm.Q[16 * mw + li][128 * g + 8 * ks]);     \
    /* sum of squares straight from the packed bf16 pairs (v_dot2) */                        \
    float ssp[4] = {0.f, 0.f, 0.f, 0.f};                                                     \
    _Pragma("unroll") for (int ks = 0; ks < 16; ++ks)                                        \
      ssp[ks & 3] = sumsq_bf16x8(qraw[ks], ssp[ks & 3]);                                     \
    float ss = (ssp[0] + ssp[1]) + (ssp[2] + ssp[3]);                                        \
    ss += __shfl_xor(ss, 16);                                                                \
    ss += __shfl_xor(ss, 32);                                                                \
    const float inv = 1.0f / sqrtf(ss / (float)AT_C + a.eps);                                \
    /* lane group 3 holds the last channels: a chunk ks can hold RoPE channels only */    \
    /* when 384 + 8 ks + 8 > c - d_r (the same test for every lane).  There every lane */    \
    /* takes the pair coefficients; elsewhere the pair form reduces to x g qscale. */        \
    _Pragma("unroll") for (int ks = 0; ks < 16; ++ks) {                                      \
      u32x4 pk;                                                                              \
      if (392 + 8 * ks > AT_C - d_r) {                                                       \
        const f32x4* c4 = &sm.qc[(128 * g + 8 * ks) >> 1];                                   \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                      \
          const f32x4 c = c4[i];                                                             \
          const float x0 = __uint_as_float(qraw[ks][i] << 16) * inv;                         \
          const float x1 = __uint_as_float(qraw[ks][i] & 0xFFFF0000u) * inv;                 \
          pk[i] = pack_bf16x2_hw(fmaf(c[0], x0, -c[1] * x1), fmaf(c[2], x0, c[3] * x1));     \
        }                                                                                    \
      } else if (a.q_norm_w != nullptr) {                                                    \
        const f32x4 ga = *reinterpret_cast<const f32x4*>(&sm.gq[128 * g + 8 * ks]);          \
        const f32x4 gb = *reinterpret_cast<const f32x4*>(&sm.gq[128 * g + 8 * ks + 4]);      \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                      \
          const f32x4 gg = i < 2 ? ga : gb;                                                  \
          const float x0 = __uint_as_float(qraw[ks][i] << 16) * inv;                         \
          const float x1 = __uint_as_float(qraw[ks][i] & 0xFFFF0000u) * inv;                 \
          pk[i] = pack_bf16x2_hw(gg[2 * (i & 1)] * x0, gg[2 * (i & 1) + 1] * x1);            \
        }                                                                                    \
      } else {                                                                               \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                      \
          const float x0 = __uint_as_float(qraw[ks][i] << 16) * inv;                         \
          const float x1 = __uint_as_float(qraw[ks][i] & 0xFFFF0000u) * inv;                 \
          pk[i] = pack_bf16x2_hw((1.f * qscale) * x0, (1.f * qscale) * x1);                  \
        }                                                                                    \
      }                                                                                      \
      *reinterpret_cast<u32x4*>(&sm.Q[16 * mw + li][128 * g + 8 * ks]) = pk;                 \
    }                                                                                        \
  } else {                                                                                   \
    float ss = 0.f;                                                                          \
    _Pragma("unroll") for (int ks = 0; ks < 16; ++ks) {                                      \
      float v[8];                                                                            \
      load8(qrow, a.q_t, 128 * g + 8 * ks, v);                                               \
      _Pragma("unroll") for (int i = 0; i < 8; ++i) ss = fmaf(v[i], v[i], ss);               \
    }                                                                                        \
    ss += __shfl_xor(ss, 16);                                                                \
    ss += __shfl_xor(ss, 32);                                                                \
    const float inv = 1.0f / sqrtf(ss / (float)AT_C + a.eps);                                \
    _Pragma("unroll") for (int ks = 0; ks < 16; ++ks) {                                      \
      float v[8];                                                                            \
      load8(qrow, a.q_t, 128 * g + 8 * ks, v);                                               \
      const f32x4* c4 = &sm.qc[(128 * g + 8 * ks) >> 1];                                     \
      u32x4 pk;                                                                              \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                        \
        const f32x4 c = c4[i];                                                               \
        const float x0 = v[2 * i] * inv, x1 = v[2 * i + 1] * inv;                            \
        pk[i] = pack_bf16x2_hw(fmaf(c[0], x0, -c[1] * x1), fmaf(c[2], x0, c[3] * x1));       \
      }                                                                                      \
      *reinterpret_cast<u32x4*>(&sm.Q[16 * mw + li][128 * g + 8 * ks]) = pk;                 \
    }                                                                                        \
  }

  // ---- loader staging: rows 8mw..8mw+7 of a tile, lane l holds dims 8l..8l+7;
  // all addresses first (empty slots read row 0 and are zeroed at commit).
  // Needs ntiles > 0; a tile past the end re-reads the last tile (it is
  // never committed).
#define CSA_STAGE(STG, OK, T)                                                                \
  {                                                                                          \
    const uint8_t* src[8];                                                                   \
    OK = 0u;                                                                                 \
    {                                                                                        \
      const int tc = (T) < ntiles ? (T) : ntiles - 1;                                        \
      const int4* sp4 = reinterpret_cast<const int4*>(&sm.slot[tc * AT_TILE + 8 * mw]);      \
      const int4 i0 = sp4[0], i1 = sp4[1];                                                   \
      /* every lane read the same ids: scalar copies keep the addresses on the SALU */    \
      const int ids[8] = {__builtin_amdgcn_readfirstlane(i0.x), __builtin_amdgcn_readfirstlane(i0.y), \
                          __builtin_amdgcn_readfirstlane(i0.z), __builtin_amdgcn_readfirstlane(i0.w), \
                          __builtin_amdgcn_readfirstlane(i1.x), __builtin_amdgcn_readfirstlane(i1.y), \
                          __builtin_amdgcn_readfirstlane(i1.z), __builtin_amdgcn_readfirstlane(i1.w)}; \
      _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                        \
        const int id = ids[i];                                                               \
        OK |= (id != -1 ? 1u : 0u) << i;                                                     \
        const bool in_kv = id >= -1;                                                         \
        const int r = id >= 0 ? id : (id == -1 ? 0 : -2 - id);                               \
        src[i] = in_kv ? kv_addr(ctx, r) : ctx.win + (int64_t)r * rb;                        \
      }                                                                                      \
    }                                                                                        \
    /* bf16 rows: lane l takes bytes 16l..16l+15; FP8 rows (576 B): lanes    */            \
    /* 0-27 the e4m3 body, 28-35 the bf16 RoPE part, the rest repeat chunk 35 */            \
    const int ch = KVF == CSA_BF16 ? lane : (lane < 36 ? lane : 35);                         \
    _Pragma("unroll") for (int i = 0; i < 8; ++i)                                            \
      STG[i] = *reinterpret_cast<const u32x4*>(src[i] + 16 * ch);                            \
  }
#define CSA_COMMIT(STG, OK, BUF)                                                             \
  {                                                                                          \
    if ((OK) == 0xFFu) {                                                                     \
      CSA_COMMIT_ROWS(STG, 0xFFu, BUF)                                                       \
    } else {                                                                                 \
      CSA_COMMIT_ROWS(STG, OK, BUF)                                                          \
    }                                                                                        \
  }
  /* (a full set of rows needs no per-row zeroing) */
#define CSA_COMMIT_ROWS(STG, OK, BUF)                                                        \
  {                                                                                          \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                          \
      const bool ok_i = ((OK) >> i) & 1u;                                                    \
      uint16_t* xr = &sm.X[BUF][xrow(8 * mw + i)][0];                                       \
      if (KVF == CSA_BF16) {                                                                 \
        *reinterpret_cast<u32x4*>(xr + 8 * lane) = ok_i ? STG[i] : u32x4{0u, 0u, 0u, 0u};   \
      } else if (lane < 28) {                                                                \
        const u32x4 lo = e4m3x8_to_bf16(STG[i][0], STG[i][1]);                               \
        const u32x4 hi = e4m3x8_to_bf16(STG[i][2], STG[i][3]);                               \
        *reinterpret_cast<u32x4*>(xr + 16 * lane) = ok_i ? lo : u32x4{0u, 0u, 0u, 0u};      \
        *reinterpret_cast<u32x4*>(xr + 16 * lane + 8) = ok_i ? hi : u32x4{0u, 0u, 0u, 0u};  \
      } else if (lane < 36) {                                                                \
        *reinterpret_cast<u32x4*>(xr + 448 + 8 * (lane - 28)) =                              \
            ok_i ? STG[i] : u32x4{0u, 0u, 0u, 0u};                                           \
      }                                                                                      \
    }                                                                                        \
  }

  // transpose-read addresses: lane (g, q = li) reads entry 8g + 4h + li/4,
  // dims 16nd + 4(li%4) .. +3
  const int tr_r0 = xrow(8 * g + (li >> 2)), tr_r1 = xrow(8 * g + 4 + (li >> 2));
  const int tr_c = 4 * (li & 3);


  if (!math && RING == 3) {
    // ---- loaders, long split lists: a ring of 3 register sets; tile u lives
    // in set u % 3 and phase u stages tile u + 3, so three tiles are in
    // flight per block while one is committed.  Same barrier count as below.
    u32x4 st0[8], st1[8], st2[8];
    uint32_t ok0 = 0u, ok1 = 0u, ok2 = 0u;
    if (ntiles > 0) {
      CSA_STAGE(st0, ok0, 0);
      CSA_STAGE(st1, ok1, 1);
      CSA_STAGE(st2, ok2, 2);
      CSA_COMMIT(st0, ok0, 0);
      CSA_STAGE(st0, ok0, 3);
    }
    __syncthreads();
#define CSA_PHASE3(STG, OK, U)                                                               \
    {                                                                                        \
      CSA_COMMIT(STG, OK, (U) & 1);                                                          \
      CSA_STAGE(STG, OK, (U) + 3);                                                           \
      __syncthreads();                                                                       \
    }
#define CSA_LAST_PHASE3(STG, OK, U)                                                          \
    if ((U) <= ntiles) {                                                                     \
      if ((U) < ntiles) CSA_COMMIT(STG, OK, (U) & 1);                                        \
      if ((U) + 3 < ntiles) CSA_STAGE(STG, OK, (U) + 3);                                     \
      __syncthreads();                                                                       \
    }
    int u = 1;
    for (; u + 5 < ntiles; u += 3) {
      CSA_PHASE3(st1, ok1, u);
      CSA_PHASE3(st2, ok2, u + 1);
      CSA_PHASE3(st0, ok0, u + 2);
    }
    CSA_LAST_PHASE3(st1, ok1, u);
    CSA_LAST_PHASE3(st2, ok2, u + 1);
    CSA_LAST_PHASE3(st0, ok0, u + 2);
    CSA_LAST_PHASE3(st1, ok1, u + 3);
    CSA_LAST_PHASE3(st2, ok2, u + 4);
    CSA_LAST_PHASE3(st0, ok0, u + 5);
#undef CSA_PHASE3
#undef CSA_LAST_PHASE3
    return;
  }
  if (!math) {
    // ---- loaders: a ring of 2 register sets; tile u lives in set u % 2.
    // While the math waves compute tile t from X[t & 1], tile t+1 is committed
    // into X[(t+1) & 1] and tile t+3 is fetched into the set it frees.  Two
    // tiles in flight per block already keep HBM busy with every CU loading,
    // and a shallower ring brings each block's first tile back sooner.  The
    // barrier count matches the math waves': one, then one per tile.
    u32x4 st0[8], st1[8];
    uint32_t ok0 = 0u, ok1 = 0u;
    if (ntiles > 0) {
      CSA_STAGE(st0, ok0, 0);
      CSA_STAGE(st1, ok1, 1);
    }
    if (ntiles > 0) {
      CSA_COMMIT(st0, ok0, 0);
      CSA_STAGE(st0, ok0, 2);
    }
    __syncthreads();
    // phase u (1 .. ntiles): commit tile u (when it exists) from set u % 2,
    // stage tile u + 2 into that set (when it exists), then the tile barrier.
    // While every stage is a real tile, phases run in pairs with one loop
    // exit and a stage in every phase, so each commit waits for its own tile
    // only; the last phases (at most four) follow with their conditions.
#define CSA_PHASE(STG, OK, U)                                                                \
    {                                                                                        \
      CSA_COMMIT(STG, OK, (U) & 1);                                                          \
      CSA_STAGE(STG, OK, (U) + 2);                                                           \
      __syncthreads();                                                                       \
    }
#define CSA_LAST_PHASE(STG, OK, U)                                                           \
    if ((U) <= ntiles) {                                                                     \
      if ((U) < ntiles) CSA_COMMIT(STG, OK, (U) & 1);                                        \
      if ((U) + 2 < ntiles) CSA_STAGE(STG, OK, (U) + 2);                                     \
      __syncthreads();                                                                       \
    }
    int u = 1;
    for (; u + 3 < ntiles; u += 2) {
      CSA_PHASE(st1, ok1, u);
      CSA_PHASE(st0, ok0, u + 1);
    }
    CSA_LAST_PHASE(st1, ok1, u);
    CSA_LAST_PHASE(st0, ok0, u + 1);
    CSA_LAST_PHASE(st1, ok1, u + 2);
    CSA_LAST_PHASE(st0, ok0, u + 3);
#undef CSA_PHASE
#undef CSA_LAST_PHASE
    return;
  }
  // this wave's queries: loads and preparation overlap the loaders' first gathers
  CSA_QPREP();
  float m_run = kNegBig, l_run = 0.f;
  f32x4 O[32];
#pragma unroll
  for (int nd = 0; nd < 32; ++nd) O[nd] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();  // tile 0 in LDS
  // this wave's query fragments (B operand of S^T), kept in registers
  bf16x8 qf[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks)
    qf[ks] = *reinterpret_cast<const bf16x8*>(&sm.Q[16 * mw + li][128 * g + 8 * ks]);
  for (int t = 0; t < ntiles; ++t) {
    CSA_TILE(t, t & 1, 3, 8);
    __syncthreads();
  }
#undef CSA_STAGE
#undef CSA_COMMIT
#undef CSA_COMMIT_ROWS
#undef CSA_QPREP

  // ---- lane holds O^T[dim 16nd + 4g + r][head]; head totals across the 4 groups
  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (nsplit == 1) {
    attend_store_out(a, row, head, g, O, m_run, l_tot, sm.rcs, &sm.Q[16 * mw][0]);
  } else {
    // partials: O / l in bf16 [rows, nsplit, nh, 512], then (m, l) fp32
    // [rows, nsplit, nh, 2].  Each split's O / l is a convex combination of
    // its rows, so bf16 costs at most 2^-9 of the largest row value.
    const int64_t rs = (int64_t)row * nsplit + split;
    const float il = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    // staged through the wave's own 16 rows of sm.Q (its queries are in
    // registers now), then written one 1 KB head row per instruction; the
    // same wave reads back what it wrote (LDS keeps its accesses in order)
#pragma unroll
    for (int nd = 0; nd < 32; ++nd)
      *reinterpret_cast<uint2*>(&sm.Q[16 * mw + li][16 * nd + 4 * g]) =
          make_uint2(pack_bf16x2_hw(O[nd][0] * il, O[nd][1] * il), pack_bf16x2_hw(O[nd][2] * il, O[nd][3] * il));
    uint16_t* wo = reinterpret_cast<uint16_t*>(ws) + (rs * a.nh + 64 * hg + 16 * mw) * AT_C;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      *reinterpret_cast<u32x4*>(wo + (int64_t)i * AT_C + 8 * lane) =
          *reinterpret_cast<const u32x4*>(&sm.Q[16 * mw + i][8 * lane]);
    if (g == 0) {
      const int64_t nrows = (int64_t)a.B * a.Tq;
      float* wml = reinterpret_cast<float*>(reinterpret_cast<uint16_t*>(ws) + nrows * nsplit * a.nh * AT_C) +
                   (rs * a.nh + head) * 2;
      wml[0] = m_run * kLn2;  // natural units for the merge
      wml[1] = l_tot;
    }
  }
}

// ============================================================ MFMA, two blocks per CU
// Many query rows over bf16 rows with bf16 queries (prefill, and short lists): one 256-thread
// block per (query row, 64 heads) over the whole slot list, two blocks
// resident per compute unit.  Each of the 4 waves owns 16 heads and also
// gathers 8 rows of every tile, straight into shared memory (global_load_lds,
// 16 bytes per lane, one tile ahead of the math).  With two blocks per CU,
// every SIMD runs two math waves of different query rows, so one wave's
// softmax, loads and barrier waits overlap the other's matrix-core work; the
// single-block kernel above has one math wave per SIMD beside a loader.
// Queries are normalised and rotated in registers (no shared copy), and empty
// slots are not loaded: their tile rows hold zeros or an earlier valid row,
// and their weights are 0.
constexpr int PF_ROPE_MAX = 64;  // RoPE dims (the rotation table is sized for these)
constexpr int PF_CHUNK = 16;     // (row, head group) items per XCD run

// One wave copies a 1 KB row into shared memory: lane l's 16 bytes at src go
// to shared address dst + 16 l (global_load_lds_dwordx4, M0 = dst).  Written as asm, which
// has no output registers, so that the compiler does not track the copy: it
// cannot tell which tile a copy writes, and would otherwise wait for every
// copy in flight before each transpose read of the other tile.  The kernel
// orders the copies itself (vmcnt(0) and a barrier before a tile is read).
__device__ __forceinline__ void pf_gather_row(const uint8_t* src, uint32_t dst) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(dst) : "memory");
}

struct AttendPfSmem {
  uint16_t X[2][AT_TILE][AT_LDX];  // gathered rows (double-buffered tiles), rows permuted by xrow
  int32_t slot[AT_TAB + 64];
  uint32_t vmask[AT_TAB / 32 + 2];
  float rcs[PF_ROPE_MAX / 2][2];   // cos / sin of the query position for each RoPE pair
};

__global__ __launch_bounds__(256, 2) void attend_pf_kernel(AttendArgs a, Rope rt, int per_xcd) {
  __shared__ __attribute__((aligned(16))) AttendPfSmem sm;
  const int hgroups = a.nh / 64;
  // (row, head group) items go to the XCDs (blocks i with i % 8 == x run on
  // XCD x) in runs of PF_CHUNK, round-robin: neighbouring query rows select
  // overlapping rows, which a run fetches into one L2, and every XCD gets a
  // share of the short early rows of a causal prefill (whole eighths of the
  // rows per XCD left the first one idle: 3% slower at 32K)
  const int xj = blockIdx.x >> 3;
  const int lin = ((xj / PF_CHUNK) * 8 + (blockIdx.x & 7)) * PF_CHUNK + xj % PF_CHUNK;
  if (lin >= a.B * a.Tq * hgroups) return;
  const int row = lin / hgroups, hg = lin % hgroups;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int head = 64 * hg + 16 * w + li;  // the head of this lane's softmax state
  const int d_r = a.rope_dims;
  const float qscale = a.scale * kLog2e;  // queries carry tau * log2 e: logits in log2 units
  const SlotCtx ctx = make_ctx(a, row);
  const int total = ctx.kslots + a.n_win;
  const int ntiles = (total + AT_TILE - 1) / AT_TILE;
  const int64_t rb = ctx.rb;

  // ---- slot table and per-tile validity masks, RoPE angles, zeroed tiles
  for (int i = tid; i < ((ntiles * AT_TILE + 63) & ~63); i += 256) {
    const int id = (i < total) ? slot_row_id(ctx, i) : -1;
    sm.slot[i] = id;
    const uint64_t bal = __ballot(id != -1);
    if (lane == 0) {
      sm.vmask[i >> 5] = (uint32_t)bal;
      sm.vmask[(i >> 5) + 1] = (uint32_t)(bal >> 32);
    }
  }
  for (int u = tid; u < d_r / 2; u += 256) {
    float cs, sn;
    rope_cs(rt, (double)ctx.qp, u, &cs, &sn);
    sm.rcs[u][0] = cs;
    sm.rcs[u][1] = sn;
  }
  for (int i = tid; i < 2 * AT_TILE * AT_LDX / 8; i += 256)
    reinterpret_cast<u32x4*>(&sm.X[0][0][0])[i] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();  // table, angles and zeroed tiles ready

  // shared address of the tile buffers, and the wave index, as scalars
  const uint32_t x_lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t*)&sm.X[0][0][0]);
  const int wu = __builtin_amdgcn_readfirstlane(w);
  // ---- gather rows 8w .. 8w+7 of tile T into X[BUF]: one 1 KB row per wave
  // instruction, lane l bytes 16l .. 16l+15; slot ids are wave-uniform scalars
#define CSA_PF_LOAD(T, BUF)                                                                  \
  {                                                                                          \
    const int4* sp4 = reinterpret_cast<const int4*>(&sm.slot[(T) * AT_TILE + 8 * w]);        \
    const int4 i0 = sp4[0], i1 = sp4[1];                                                     \
    const int ids[8] = {__builtin_amdgcn_readfirstlane(i0.x), __builtin_amdgcn_readfirstlane(i0.y), \
                        __builtin_amdgcn_readfirstlane(i0.z), __builtin_amdgcn_readfirstlane(i0.w), \
                        __builtin_amdgcn_readfirstlane(i1.x), __builtin_amdgcn_readfirstlane(i1.y), \
                        __builtin_amdgcn_readfirstlane(i1.z), __builtin_amdgcn_readfirstlane(i1.w)}; \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                          \
      const int id = ids[i];                                                                 \
      if (id != -1) {                                                                        \
        const uint8_t* src = id >= 0 ? kv_addr(ctx, id) : ctx.win + (int64_t)(-2 - id) * rb;  \
        pf_gather_row(src + 16 * lane,                                                       \
                      x_lds + (uint32_t)(((BUF) * AT_TILE + xrow(8 * wu + i)) * (AT_LDX * 2))); \
      }                                                                                      \
    }                                                                                        \
  }
  if (ntiles > 0) CSA_PF_LOAD(0, 0);

  // ---- queries (B operand of S^T) in registers: raw dims 128g .. 128g+127 of
  // this lane's head, RMSNorm over the head (its four lane groups), RoPE at q,
  // scaled to log2 units, bf16
  const uint8_t* qrow = (const uint8_t*)a.q + ((int64_t)row * a.nh + head) * row_bytes(a.q_t, AT_C, 0);
  u32x4 qraw[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) qraw[ks] = *reinterpret_cast<const u32x4*>(qrow + 2 * (128 * g + 8 * ks));
  bf16x8 qf[16];
  {
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(qraw[ks][i] << 16);
        v[2 * i + 1] = __uint_as_float(qraw[ks][i] & 0xFFFF0000u);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(v[i], v[i], ss);
    }
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    const float inv = 1.0f / sqrtf(ss / (float)AT_C + a.eps);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const int d0 = 128 * g + 8 * ks;
      float v[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(qraw[ks][i] << 16);
        v[2 * i + 1] = __uint_as_float(qraw[ks][i] & 0xFFFF0000u);
      }
      if (a.q_norm_w != nullptr) {
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(a.q_norm_w + d0);
        const f32x4 g1 = *reinterpret_cast<const f32x4*>(a.q_norm_w + d0 + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] *= inv * g0[i];
          v[4 + i] *= inv * g1[i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] *= inv;
      }
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const int d = d0 + i;
        if (d >= AT_C - d_r) {
          const float cs = sm.rcs[(d - (AT_C - d_r)) >> 1][0];
          const float sn = sm.rcs[(d - (AT_C - d_r)) >> 1][1];
          const float x0 = v[i], x1 = v[i + 1];
          v[i] = x0 * cs - x1 * sn;
          v[i + 1] = x0 * sn + x1 * cs;
        }
      }
      u32x4 pk;
#pragma unroll
      for (int i = 0; i < 4; ++i) pk[i] = pack_bf16x2_hw(v[2 * i] * qscale, v[2 * i + 1] * qscale);
      qf[ks] = __builtin_bit_cast(bf16x8, pk);
    }
  }

  float m_run = kNegBig, l_run = 0.f;
  f32x4 O[32];
#pragma unroll
  for (int nd = 0; nd < 32; ++nd) O[nd] = f32x4{0.f, 0.f, 0.f, 0.f};
  // transpose-read addresses: lane (g, q = li) reads entry 8g + 4h + li/4,
  // dims 16nd + 4(li%4) .. +3
  const int tr_r0 = xrow(8 * g + (li >> 2)), tr_r1 = xrow(8 * g + 4 + (li >> 2));
  const int tr_c = 4 * (li & 3);
  for (int t = 0; t < ntiles; ++t) {
    // this wave's rows of tile t have landed; after the barrier every wave's
    // have, and every wave is done with tile t-1, whose buffer takes tile t+1
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (t + 1 < ntiles) CSA_PF_LOAD(t + 1, (t + 1) & 1);
    CSA_TILE(t, t & 1, 2, 4);
  }
#undef CSA_PF_LOAD
  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16);
  l_tot += __shfl_xor(l_tot, 32);
  // every wave is done with the last tile: the tile buffers stage the output
  // (wave w takes rows 16 w .. 16 w + 15 of the 64)
  __syncthreads();
  attend_store_out(a, row, head, g, O, m_run, l_tot, sm.rcs, &sm.X[0][0][0] + 16 * w * AT_LDX);
}
#undef CSA_TILE

// merge split partials in split order, add the sink, normalise, inverse RoPE;
// one block per (query row, head), one thread per channel pair
__global__ __launch_bounds__(256) void attend_combine_kernel(AttendArgs a, Rope rt,
                                                             int nsplit,
                                                             const void* __restrict__ ws) {
  const int nh = a.nh, c = a.c, d_r = a.rope_dims;
  // the XCD that wrote row r's partials (r % 8) merges them
  const int xj = blockIdx.x >> 3;
  const int row = (xj / nh) * 8 + (blockIdx.x & 7), h = xj % nh;
  const int d = 2 * threadIdx.x;
  const int64_t nrows = (int64_t)a.B * a.Tq;
  if (d >= c || row >= nrows) return;
  const uint16_t* wo = reinterpret_cast<const uint16_t*>(ws) + (int64_t)row * nsplit * nh * c;
  const float* wml = reinterpret_cast<const float*>(reinterpret_cast<const uint16_t*>(ws) +
                                                    nrows * nsplit * nh * c) +
                     (int64_t)row * nsplit * nh * 2;
  const float z = a.sink[h];
  float M = z, den, o0 = 0.f, o1 = 0.f;
  if (nsplit <= 16) {
    // every split's (m, l) and partial requested at once, then merged in
    // split order (the same arithmetic as the general loop below)
    float2 ml[16];
    uint32_t v[16];
#pragma unroll
    for (int s = 0; s < 16; ++s)
      if (s < nsplit) {
        ml[s] = *reinterpret_cast<const float2*>(wml + ((int64_t)s * nh + h) * 2);
        v[s] = *reinterpret_cast<const uint32_t*>(wo + ((int64_t)s * nh + h) * c + d);
      }
#pragma unroll
    for (int s = 0; s < 16; ++s)
      if (s < nsplit) M = fmaxf(M, ml[s].x);
    den = __expf(z - M);
#pragma unroll
    for (int s = 0; s < 16; ++s)
      if (s < nsplit) {
        const float wgt = ml[s].y * __expf(ml[s].x - M);
        den += wgt;
        o0 = fmaf(__uint_as_float(v[s] << 16), wgt, o0);
        o1 = fmaf(__uint_as_float(v[s] & 0xFFFF0000u), wgt, o1);
      }
  } else {
#pragma unroll 8
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, wml[((int64_t)s * nh + h) * 2]);
    den = __expf(z - M);
#pragma unroll 8
    for (int s = 0; s < nsplit; ++s) {
      const float wgt = wml[((int64_t)s * nh + h) * 2 + 1] * __expf(wml[((int64_t)s * nh + h) * 2] - M);
      den += wgt;
      const uint32_t v = *reinterpret_cast<const uint32_t*>(wo + ((int64_t)s * nh + h) * c + d);
      o0 = fmaf(__uint_as_float(v << 16), wgt, o0);
      o1 = fmaf(__uint_as_float(v & 0xFFFF0000u), wgt, o1);
    }
  }
  const float inv = 1.0f / den;
  o0 *= inv;
  o1 *= inv;
  if (d >= c - d_r) {
    float cs, sn;
    rope_cs(rt, -(double)a.q_pos[row], (d - (c - d_r)) >> 1, &cs, &sn);
    const float x0 = o0, x1 = o1;
    o0 = x0 * cs - x1 * sn;
    o1 = x0 * sn + x1 * cs;
  }
  const int64_t ob = ((int64_t)row * nh + h) * c + d;
  if (a.out_t == CSA_F32) {
    reinterpret_cast<float2*>(a.out)[ob / 2] = make_float2(o0, o1);
  } else {
    reinterpret_cast<uint32_t*>(a.out)[ob / 2] = pack_bf16x2(o0, o1);
  }
}

// ============================================================ dispatch
static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

static bool use_mfma(const AttendArgs& a) {
  // FP8 rows are staged as 448 e4m3 + 64 bf16 bytes: RoPE on the last 64.
  // Queries, rows and outputs move in 16-byte pieces.
  return a.c == AT_C && a.nh % 64 == 0 && (a.kv_t == CSA_BF16 || a.kv_t == CSA_FP8MIX) &&
         (a.q_t == CSA_BF16 || a.q_t == CSA_F32) && a.rope_dims % 2 == 0 && a.rope_dims <= AT_C &&
         (a.kv_t != CSA_FP8MIX || a.rope_dims == 64) && aligned16(a.q) && aligned16(a.kv) &&
         aligned16(a.win) && aligned16(a.out);
}

// slot split: a function of the per-row slot count only (never of the batch
// size), so a sequence's result does not depend on what else is in the batch;
// long lists of few query rows split, many query rows never do
static void plan_splits(const AttendArgs& a, int* chunk, int* nsplit) {
  const int kslots = a.idx ? a.k : a.Nmax;
  const int total = kslots + a.n_win;
  if ((a.Tq > 1 || total <= 256) && total <= AT_TAB) {
    *chunk = ((total + AT_TILE - 1) / AT_TILE) * AT_TILE;
    *nsplit = 1;
    return;
  }
  // 8 splits per 64-head group up to 4096 slots (at most 16), 16 beyond: a
  // decode batch of 8 rows x 128 heads or 32 rows x 64 heads then gives about
  // one block per compute unit.  Splits are whole tiles, at least 3.
  const int hgroups = a.nh / 64;
  const int want = total <= 4096 ? (hgroups > 1 ? 16 : 8) : 16;
  int ch = ((total + want - 1) / want + AT_TILE - 1) / AT_TILE * AT_TILE;
  ch = ch < 3 * AT_TILE ? 3 * AT_TILE : (ch > AT_TAB ? AT_TAB : ch);
  *chunk = ch;
  *nsplit = (total + ch - 1) / ch;
}

size_t attend_workspace(const AttendArgs& a) {
  if (!use_mfma(a)) return 0;
  int chunk, nsplit;
  plan_splits(a, &chunk, &nsplit);
  if (nsplit == 1) return 0;
  const size_t rows = (size_t)a.B * a.Tq;
  return rows * nsplit * a.nh * ((size_t)a.c * sizeof(uint16_t) + 2 * sizeof(float));
}

hipError_t launch_attend(const AttendArgs& a, void* ws, hipStream_t s) {
  const int rows = a.B * a.Tq;
  if (rows == 0) return hipSuccess;
  const Rope rt = make_rope(a.rope_dims, a.rope_theta);
  if (!use_mfma(a)) {
    const int nw = a.nh < 4 ? a.nh : 4;
    const size_t shm = (size_t)nw * a.c * sizeof(float);
    if (a.c <= 64)
      hipLaunchKernelGGL(attend_generic_kernel<1>, dim3(rows), dim3(64 * nw), shm, s, a, rt);
    else if (a.c <= 128)
      hipLaunchKernelGGL(attend_generic_kernel<2>, dim3(rows), dim3(64 * nw), shm, s, a, rt);
    else if (a.c <= 512)
      hipLaunchKernelGGL(attend_generic_kernel<8>, dim3(rows), dim3(64 * nw), shm, s, a, rt);
    else
      hipLaunchKernelGGL(attend_generic_kernel<16>, dim3(rows), dim3(64 * nw), shm, s, a, rt);
    return hipGetLastError();
  }
  int chunk, nsplit;
  plan_splits(a, &chunk, &nsplit);
  if (nsplit == 1 && a.kv_t == CSA_BF16 && a.q_t == CSA_BF16 && a.rope_dims <= PF_ROPE_MAX) {
    // one block per (query row, 64 heads), two resident per compute unit
    const int64_t nb = (int64_t)rows * (a.nh / 64);
    // blocks per XCD: whole runs of PF_CHUNK (items past the end exit)
    const int per_xcd = (int)((nb + 8 * PF_CHUNK - 1) / (8 * PF_CHUNK) * PF_CHUNK);
    hipLaunchKernelGGL(attend_pf_kernel, dim3((unsigned)(8 * (int64_t)per_xcd)), dim3(256), 0, s, a, rt,
                       per_xcd);
    return hipGetLastError();
  }
  // rows rounded up to a multiple of 8 for the XCD-aware block order
  const int64_t rows8 = (rows + 7) / 8 * 8;
  dim3 grid((unsigned)((int64_t)nsplit * (a.nh / 64) * rows8));
  void* w = ws;
  const bool qb = a.q_t == CSA_BF16;
  // splits of 8 tiles or more (long dense lists) keep three tiles in flight
  if (a.kv_t == CSA_BF16 && qb && chunk >= 8 * AT_TILE)
    hipLaunchKernelGGL((attend_mfma_kernel<CSA_BF16, true, 3>), grid, dim3(512), 0, s, a, rt, chunk, nsplit, w);
  else if (a.kv_t == CSA_BF16 && qb)
    hipLaunchKernelGGL((attend_mfma_kernel<CSA_BF16, true, 2>), grid, dim3(512), 0, s, a, rt, chunk, nsplit, w);
  else if (a.kv_t == CSA_BF16)
    hipLaunchKernelGGL((attend_mfma_kernel<CSA_BF16, false, 2>), grid, dim3(512), 0, s, a, rt, chunk, nsplit, w);
  else if (qb)
    hipLaunchKernelGGL((attend_mfma_kernel<CSA_FP8MIX, true, 2>), grid, dim3(512), 0, s, a, rt, chunk, nsplit, w);
  else
    hipLaunchKernelGGL((attend_mfma_kernel<CSA_FP8MIX, false, 2>), grid, dim3(512), 0, s, a, rt, chunk, nsplit, w);
  if (nsplit > 1)
    hipLaunchKernelGGL(attend_combine_kernel, dim3((unsigned)(rows8 * a.nh)),
                       dim3((a.c / 2 + 63) / 64 * 64), 0, s, a, rt, nsplit, (const void*)w);
  return hipGetLastError();
}

}  // namespace csa
