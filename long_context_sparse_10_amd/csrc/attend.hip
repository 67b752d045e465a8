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
//  * attend_mfma_kernel   -- c = 512, heads a multiple of 16, bf16 or
//    FP8/BF16 KV.  One block per (query row, slot split); wave w owns heads
//    16w..16w+15 with its RMSNorm'd, RoPE'd query held as bf16 MFMA fragments.
//    32-slot tiles of KV rows are gathered into LDS (double buffered, e4m3
//    expanded to bf16 on the way), S = Q K^T and O += P V run on
//    v_mfma_f32_16x16x32_bf16 with an fp32 online softmax in registers.
//    With one split the block finishes the output itself; otherwise it writes
//    (m, l, O) partials and attend_combine_kernel merges the splits in order.
//  * attend_generic_kernel -- any shape / fp32: one wave per head, VALU.
#include "common.hpp"
#include "internal.hpp"

namespace csa {

constexpr float kNegBig = -3.0e38f;  // finite "minus infinity" for running maxima

struct SlotCtx {
  const uint8_t* kv;
  const uint8_t* win;
  const int32_t* idx_row;  // sparse only
  int64_t kv_base;         // b * Nmax
  int64_t win_base;        // b * win_len
  int64_t rb;              // bytes per row
  int kslots, nv, qp, n_win, win_len, nmax;
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
      return kv + (kv_base + s) * rb;
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
  x.kv_base = (int64_t)b * a.Nmax;
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
__global__ __launch_bounds__(256) void attend_generic_kernel(AttendArgs a) {
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
      rope_cs((double)ctx.qp, u, d_r, a.rope_theta, &cs, &sn);
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
        rope_cs(-(double)ctx.qp, u, d_r, a.rope_theta, &cs, &sn);
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
constexpr int AT_LDX = AT_C + 8;  // bf16 per LDS row; 16-byte pad

template <int KVF, int NW>
struct AttendSmem {
  uint16_t X[2][AT_TILE][AT_LDX];
  uint16_t P[NW][16][AT_TILE + 8];
  int valid[2][AT_TILE];
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

template <int KVF, int NW>
__global__ __launch_bounds__(NW * 64) void attend_mfma_kernel(AttendArgs a, int chunk,
                                                             int nsplit, float* __restrict__ ws) {
  __shared__ __attribute__((aligned(16))) AttendSmem<KVF, NW> sm;
  // block -> (query row, head group of 16*NW heads, slot split)
  const int hgroups = a.nh / (16 * NW);
  const int split = blockIdx.x % nsplit;
  const int hg = (blockIdx.x / nsplit) % hgroups;
  const int row = blockIdx.x / (nsplit * hgroups);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int hbase = 16 * NW * hg + 16 * wave;  // first head of this wave
  const int d_r = a.rope_dims;
  const SlotCtx ctx = make_ctx(a, row);
  const int total = ctx.kslots + a.n_win;
  const int v0 = split * chunk;
  const int v1 = min(v0 + chunk, total);
  const int ntiles = v1 > v0 ? (v1 - v0 + AT_TILE - 1) / AT_TILE : 0;

  // ---- query fragments: head 16*wave + li, physical dims 128*g + 8*ks + 0..7
  bf16x8 qf[16];
  {
    const int head = hbase + li;
    const uint8_t* qrow = (const uint8_t*)a.q + ((int64_t)row * a.nh + head) * row_bytes(a.q_t, AT_C, 0);
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      float v[8];
      load8(qrow, a.q_t, 128 * g + 8 * ks, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) ss = fmaf(v[j], v[j], ss);
    }
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    const float inv = 1.0f / sqrtf(ss / (float)AT_C + a.eps);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const int d0 = 128 * g + 8 * ks;
      float v[8];
      load8(qrow, a.q_t, d0, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] *= inv * (a.q_norm_w ? a.q_norm_w[d0 + j] : 1.f);
      if (d0 + 8 > AT_C - d_r) {
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const int d = d0 + j;
          if (d >= AT_C - d_r) {
            float cs, sn;
            rope_cs((double)ctx.qp, (d - (AT_C - d_r)) >> 1, d_r, a.rope_theta, &cs, &sn);
            const float x0 = v[j], x1 = v[j + 1];
            v[j] = x0 * cs - x1 * sn;
            v[j + 1] = x0 * sn + x1 * cs;
          }
        }
      }
      u32x4 pk;
#pragma unroll
      for (int i = 0; i < 4; ++i) pk[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
      qf[ks] = __builtin_bit_cast(bf16x8, pk);
    }
  }

  // ---- tile staging: each wave gathers rows wave, wave+NW, ... of a tile
  constexpr int RPW = AT_TILE / NW;
  u32x4 stg[RPW];
  int stg_ok[RPW];
  auto stage = [&](int t) {
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int rr = wave + NW * i;
      const int v = v0 + t * AT_TILE + rr;
      const uint8_t* src = (v < v1) ? ctx.row(v) : nullptr;
      stg_ok[i] = src != nullptr;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (src != nullptr) {
        if (KVF == CSA_BF16) {
          val = *reinterpret_cast<const u32x4*>(src + 16 * lane);
        } else {  // FP8MIX: 448 e4m3 bytes (lanes 0..27) then 64 bf16 (lanes 28..35)
          if (lane < 36) val = *reinterpret_cast<const u32x4*>(src + 16 * lane);
        }
      }
      stg[i] = val;
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int rr = wave + NW * i;
      uint16_t* dst = &sm.X[buf][rr][0];
      if (KVF == CSA_BF16) {
        *reinterpret_cast<u32x4*>(dst + 8 * lane) = stg[i];
      } else {
        if (lane < 28) {  // 16 e4m3 -> 16 bf16 (exact)
          u32x4 lo, hi;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t wv = stg[i][q];
            const float f0 = e4m3_to_f32(wv & 0xFFu), f1 = e4m3_to_f32((wv >> 8) & 0xFFu);
            const float f2 = e4m3_to_f32((wv >> 16) & 0xFFu), f3 = e4m3_to_f32(wv >> 24);
            const uint32_t p0 = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xFFFF0000u);
            const uint32_t p1 = (__float_as_uint(f2) >> 16) | (__float_as_uint(f3) & 0xFFFF0000u);
            if (q < 2) { lo[2 * q] = p0; lo[2 * q + 1] = p1; }
            else { hi[2 * q - 4] = p0; hi[2 * q - 3] = p1; }
          }
          *reinterpret_cast<u32x4*>(dst + 16 * lane) = lo;
          *reinterpret_cast<u32x4*>(dst + 16 * lane + 8) = hi;
        } else if (lane < 36) {
          *reinterpret_cast<u32x4*>(dst + 448 + 8 * (lane - 28)) = stg[i];
        }
      }
      if (lane == 0) sm.valid[buf][rr] = stg_ok[i];
    }
  };

  float m_run[4], l_run[4];
  f32x4 O[32];
#pragma unroll
  for (int r = 0; r < 4; ++r) { m_run[r] = kNegBig; l_run[r] = 0.f; }
#pragma unroll
  for (int nd = 0; nd < 32; ++nd) O[nd] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (ntiles > 0) {
    stage(0);
    commit(0);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) stage(t + 1);
    int any = 0;
#pragma unroll
    for (int e = 0; e < AT_TILE; ++e) any |= sm.valid[buf][e];
    if (any) {
      // S = Q K^T : two 16-entry sub-tiles, K = 512 in 16 steps
      f32x4 S[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        S[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const uint16_t* xr = &sm.X[buf][16 * nt + li][128 * g];
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
          const bf16x8 kb = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xr + 8 * ks));
          S[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ks], kb, S[nt], 0, 0, 0);
        }
      }
      // online softmax; lane holds heads 4g+r for entries 16nt+li
      const int ok0 = sm.valid[buf][li], ok1 = sm.valid[buf][16 + li];
      float p0[4], p1[4], alpha[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float l0 = ok0 ? a.scale * S[0][r] : -INFINITY;
        const float l1 = ok1 ? a.scale * S[1][r] : -INFINITY;
        float mx = fmaxf(l0, l1);
        mx = fmaxf(mx, __shfl_xor(mx, 1));
        mx = fmaxf(mx, __shfl_xor(mx, 2));
        mx = fmaxf(mx, __shfl_xor(mx, 4));
        mx = fmaxf(mx, __shfl_xor(mx, 8));
        const float m_new = fmaxf(m_run[r], mx);
        alpha[r] = __expf(m_run[r] - m_new);
        p0[r] = __expf(l0 - m_new);
        p1[r] = __expf(l1 - m_new);
        l_run[r] = l_run[r] * alpha[r] + p0[r] + p1[r];
        m_run[r] = m_new;
      }
#pragma unroll
      for (int nd = 0; nd < 32; ++nd)
#pragma unroll
        for (int r = 0; r < 4; ++r) O[nd][r] *= alpha[r];
      // P (bf16) through LDS into the A-operand layout: head li, entries 8g..8g+7
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sm.P[wave][4 * g + r][li] = (uint16_t)f32_to_bf16(p0[r]);
        sm.P[wave][4 * g + r][16 + li] = (uint16_t)f32_to_bf16(p1[r]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      const bf16x8 pf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sm.P[wave][li][8 * g]));
      // O += P V : V^T fragment = dim 16nd+li, entries 8g..8g+7 (column reads)
#pragma unroll
      for (int nd = 0; nd < 32; ++nd) {
        const uint16_t* xc = &sm.X[buf][8 * g][16 * nd + li];
        u32x4 vb;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          vb[i] = (uint32_t)xc[(2 * i) * AT_LDX] | ((uint32_t)xc[(2 * i + 1) * AT_LDX] << 16);
        O[nd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf, __builtin_bit_cast(bf16x8, vb), O[nd], 0, 0, 0);
      }
      __builtin_amdgcn_wave_barrier();
    }
    if (t + 1 < ntiles) commit(buf ^ 1);
    __syncthreads();
  }

  // ---- per-head totals over the 16 lanes of a row group
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float l = l_run[r];
    l += __shfl_xor(l, 1);
    l += __shfl_xor(l, 2);
    l += __shfl_xor(l, 4);
    l += __shfl_xor(l, 8);
    l_run[r] = l;
  }
  if (nsplit == 1) {
    // finish: sink in the denominator, normalise, inverse RoPE, store
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int head = hbase + 4 * g + r;
      const float z = a.sink[head];
      const float M = fmaxf(m_run[r], z);
      const float em = __expf(m_run[r] - M);
      const float f = em / (l_run[r] * em + __expf(z - M));
      uint8_t* orow = (uint8_t*)a.out + ((int64_t)row * a.nh + head) * row_bytes(a.out_t, AT_C, 0);
#pragma unroll
      for (int nd = 0; nd < 32; ++nd) {
        const int d = 16 * nd + li;
        float val = O[nd][r] * f;
        if (16 * nd + 16 > AT_C - d_r) {
          const float other = __shfl_xor(val, 1);
          if (d >= AT_C - d_r) {
            float cs, sn;
            rope_cs(-(double)ctx.qp, (d - (AT_C - d_r)) >> 1, d_r, a.rope_theta, &cs, &sn);
            val = (d & 1) ? other * sn + val * cs : val * cs - other * sn;
          }
        }
        if (a.out_t == CSA_F32) reinterpret_cast<float*>(orow)[d] = val;
        else reinterpret_cast<uint16_t*>(orow)[d] = (uint16_t)f32_to_bf16(val);
      }
    }
  } else {
    // partials: O [rows, nsplit, nh, 512] then (m, l) [rows, nsplit, nh, 2]
    const int64_t rs = (int64_t)row * nsplit + split;
    float* wo = ws + rs * a.nh * AT_C;
    const int64_t nrows = (int64_t)a.B * a.Tq;
    float* wml = ws + nrows * nsplit * a.nh * AT_C + rs * a.nh * 2;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int head = hbase + 4 * g + r;
#pragma unroll
      for (int nd = 0; nd < 32; ++nd) wo[(int64_t)head * AT_C + 16 * nd + li] = O[nd][r];
      if (li == 0) {
        wml[2 * head] = m_run[r];
        wml[2 * head + 1] = l_run[r];
      }
    }
  }
}

// merge split partials in split order, add the sink, normalise, inverse RoPE
__global__ __launch_bounds__(256) void attend_combine_kernel(AttendArgs a, int nsplit,
                                                             const float* __restrict__ ws) {
  const int row = blockIdx.x;
  const int c = a.c, d_r = a.rope_dims, nh = a.nh;
  const int qp = a.q_pos[row];
  const float* wo = ws + (int64_t)row * nsplit * nh * c;
  const float* wml = ws + (int64_t)gridDim.x * nsplit * nh * c + (int64_t)row * nsplit * nh * 2;
  const int pairs = c / 2;
  for (int it = threadIdx.x; it < nh * pairs; it += blockDim.x) {
    const int h = it / pairs, d = 2 * (it % pairs);
    const float z = a.sink[h];
    float M = z;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, wml[((int64_t)s * nh + h) * 2]);
    float den = __expf(z - M), o0 = 0.f, o1 = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const float e = __expf(wml[((int64_t)s * nh + h) * 2] - M);
      den = fmaf(wml[((int64_t)s * nh + h) * 2 + 1], e, den);
      const float* op = wo + ((int64_t)s * nh + h) * c + d;
      o0 = fmaf(op[0], e, o0);
      o1 = fmaf(op[1], e, o1);
    }
    o0 /= den;
    o1 /= den;
    if (d >= c - d_r) {
      float cs, sn;
      rope_cs(-(double)qp, (d - (c - d_r)) >> 1, d_r, a.rope_theta, &cs, &sn);
      const float x0 = o0, x1 = o1;
      o0 = x0 * cs - x1 * sn;
      o1 = x0 * sn + x1 * cs;
    }
    const int64_t ob = ((int64_t)row * nh + h) * c + d;
    if (a.out_t == CSA_F32) {
      reinterpret_cast<float*>(a.out)[ob] = o0;
      reinterpret_cast<float*>(a.out)[ob + 1] = o1;
    } else {
      reinterpret_cast<uint32_t*>(a.out)[ob / 2] = pack_bf16x2(o0, o1);
    }
  }
}

// ============================================================ dispatch
static bool use_mfma(const AttendArgs& a) {
  return a.c == AT_C && a.nh % 64 == 0 && (a.kv_t == CSA_BF16 || a.kv_t == CSA_FP8MIX) &&
         (a.q_t == CSA_BF16 || a.q_t == CSA_F32) && a.rope_dims % 2 == 0 && a.rope_dims <= AT_C;
}

// slot split: a function of the per-row slot count only (never of the batch
// size), so a sequence's result does not depend on what else is in the batch;
// long lists of few query rows split, many query rows never do
static void plan_splits(const AttendArgs& a, int* chunk, int* nsplit) {
  const int kslots = a.idx ? a.k : a.Nmax;
  const int total = kslots + a.n_win;
  if (a.Tq > 1 || total <= 256) {
    *chunk = ((total + AT_TILE - 1) / AT_TILE) * AT_TILE;
    *nsplit = 1;
    return;
  }
  int ch = ((total / 16 + AT_TILE - 1) / AT_TILE) * AT_TILE;
  ch = ch < 128 ? 128 : (ch > 1024 ? 1024 : ch);
  *chunk = ch;
  *nsplit = (total + ch - 1) / ch;
}

size_t attend_workspace(const AttendArgs& a) {
  if (!use_mfma(a)) return 0;
  int chunk, nsplit;
  plan_splits(a, &chunk, &nsplit);
  if (nsplit == 1) return 0;
  const size_t rows = (size_t)a.B * a.Tq;
  return rows * nsplit * a.nh * ((size_t)a.c + 2) * sizeof(float);
}

hipError_t launch_attend(const AttendArgs& a, void* ws, hipStream_t s) {
  const int rows = a.B * a.Tq;
  if (rows == 0) return hipSuccess;
  if (!use_mfma(a)) {
    const int nw = a.nh < 4 ? a.nh : 4;
    const size_t shm = (size_t)nw * a.c * sizeof(float);
    if (a.c <= 64)
      hipLaunchKernelGGL(attend_generic_kernel<1>, dim3(rows), dim3(64 * nw), shm, s, a);
    else if (a.c <= 128)
      hipLaunchKernelGGL(attend_generic_kernel<2>, dim3(rows), dim3(64 * nw), shm, s, a);
    else if (a.c <= 512)
      hipLaunchKernelGGL(attend_generic_kernel<8>, dim3(rows), dim3(64 * nw), shm, s, a);
    else
      hipLaunchKernelGGL(attend_generic_kernel<16>, dim3(rows), dim3(64 * nw), shm, s, a);
    return hipGetLastError();
  }
  int chunk, nsplit;
  plan_splits(a, &chunk, &nsplit);
  dim3 grid((unsigned)((int64_t)nsplit * (a.nh / 64) * rows));
  float* w = (float*)ws;
#define CSA_LAUNCH(KVF, NW) \
  hipLaunchKernelGGL((attend_mfma_kernel<KVF, NW>), grid, dim3(NW * 64), 0, s, a, chunk, nsplit, w)
  if (a.kv_t == CSA_BF16) CSA_LAUNCH(CSA_BF16, 4);
  else CSA_LAUNCH(CSA_FP8MIX, 4);
#undef CSA_LAUNCH
  if (nsplit > 1)
    hipLaunchKernelGGL(attend_combine_kernel, dim3(rows), dim3(256), 0, s, a, nsplit, (const float*)w);
  return hipGetLastError();
}

}  // namespace csa
