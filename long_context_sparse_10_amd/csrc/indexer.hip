// Lightning indexer (Evidence Ledger Eqs 13-17; shuhuayu section 03 score):
//   score(t, s) = sum_h w[t, h] * ReLU(qI[t, h] . kI[s])   for s < N(q_t).
//
// Hot shape (cI = 128, nI = 64, bf16 or MXFP4): the q.k contraction runs on
// v_mfma_f32_32x32x16_bf16 with the 64 heads as the M dimension (two 32-row
// tiles) and 32 entries per wave as N, K = 128.  Each lane then holds one
// entry column and 16 head rows of each tile, so the ReLU-weighted head
// reduction is 32 in-register FMAs plus one exchange with the lane 32 apart.
// Index keys stream straight from HBM into MFMA operand registers: the K order
// inside an MFMA is free, so lane half h takes 128 (bf16) or 32 (MXFP4)
// contiguous bytes of its entry's row and the query fragments use the same
// permutation.  MXFP4 codes are expanded to bf16 in registers (exact: an E2M1
// value times a power of two has at most two significant bits).
#include "common.hpp"
#include "internal.hpp"

namespace csa {

// ------------------------------------------------------------------ generic
// any nI, cI; one thread per entry, the query (dequantised) staged in LDS
__device__ __forceinline__ float load_index_elem(const uint8_t* row, const uint8_t* scales,
                                                 csa_dtype t, int j) {
  if (t == CSA_F32) return reinterpret_cast<const float*>(row)[j];
  if (t == CSA_BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(row)[j]);
  const uint32_t byte = row[j >> 1];
  const uint32_t code = (j & 1) ? (byte >> 4) : (byte & 15u);
  return e2m1_to_f32(code) * exp2i((int)scales[j >> 5] - 127);
}

__global__ __launch_bounds__(256) void indexer_generic_kernel(
    const uint8_t* __restrict__ qI, const uint8_t* __restrict__ qI_scale, csa_dtype t,
    const float* __restrict__ w, const uint8_t* __restrict__ kI, const uint8_t* __restrict__ kI_scale,
    const int32_t* __restrict__ q_pos, const int32_t* __restrict__ n_entries, int Tq, int nI,
    int cI, int Nmax, int m, void* __restrict__ scores, int score_bf16) {
  extern __shared__ float sq[];  // [nI * cI] query, then [nI] weights
  const int tiles = (Nmax + blockDim.x - 1) / blockDim.x;
  const int row = blockIdx.x / tiles, tile = blockIdx.x % tiles, b = row / Tq;
  const int nv = min(min(n_entries[b], Nmax), (q_pos[row] + 1) / m);
  if (tile * (int)blockDim.x >= nv) return;
  const int64_t qrb = row_bytes(t, cI, 0);
  for (int i = threadIdx.x; i < nI * cI; i += blockDim.x) {
    const int h = i / cI, j = i % cI;
    const int64_t qr = (int64_t)row * nI + h;
    sq[i] = load_index_elem(qI + qr * qrb, qI_scale ? qI_scale + qr * (cI / 32) : nullptr, t, j);
  }
  for (int h = threadIdx.x; h < nI; h += blockDim.x) sq[nI * cI + h] = w[(int64_t)row * nI + h];
  __syncthreads();
  const int s = tile * blockDim.x + threadIdx.x;
  if (s >= nv) return;
  const int64_t kr = (int64_t)b * Nmax + s;
  const uint8_t* krow = kI + kr * qrb;
  const uint8_t* ksc = kI_scale ? kI_scale + kr * (cI / 32) : nullptr;
  float score = 0.f;
  for (int h = 0; h < nI; ++h) {
    float dot = 0.f;
    for (int j = 0; j < cI; ++j) dot = fmaf(sq[h * cI + j], load_index_elem(krow, ksc, t, j), dot);
    score = fmaf(sq[nI * cI + h], fmaxf(dot, 0.f), score);
  }
  const int64_t o = (int64_t)row * Nmax + s;
  if (score_bf16)
    reinterpret_cast<uint16_t*>(scores)[o] = (uint16_t)f32_to_bf16(score);
  else
    reinterpret_cast<float*>(scores)[o] = score;
}

// ------------------------------------------------------------------ MFMA (nI 64, cI 128)
// 8 packed E2M1 codes (one dword, even element in the low nibble) -> 8 bf16
__device__ __forceinline__ bf16x8 e2m1x8_to_bf16(uint32_t word, float scale) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = e2m1_to_f32((word >> (8 * i)) & 15u) * scale;
    const float hi = e2m1_to_f32((word >> (8 * i + 4)) & 15u) * scale;
    r[i] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);  // exact
  }
  return __builtin_bit_cast(bf16x8, r);
}

constexpr int IDX_WAVES = 4;
constexpr int IDX_SUB = 32;  // entries per wave sub-tile

template <bool MX>
__global__ __launch_bounds__(IDX_WAVES * 64) void indexer_mfma_kernel(
    const uint8_t* __restrict__ qI, const uint8_t* __restrict__ qI_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ kI,
    const uint8_t* __restrict__ kI_scale, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_entries, int Tq, int Nmax, int m, int ent_per_block,
    void* __restrict__ scores, int score_bf16) {
  const int tiles = (Nmax + ent_per_block - 1) / ent_per_block;
  const int row = blockIdx.x / tiles, b = row / Tq;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int nv = min(min(n_entries[b], Nmax), (q_pos[row] + 1) / m);
  const int e0 = (blockIdx.x % tiles) * ent_per_block;
  if (e0 >= nv) return;
  const int e1 = min(e0 + ent_per_block, nv);

  // query fragments: head 32*mt + col, physical dims 64*half + 8*ks + 0..7
  bf16x8 afr[2][8];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int head = 32 * mt + col;
    if (!MX) {
      const u32x4* p = reinterpret_cast<const u32x4*>(qI + ((int64_t)row * 64 + head) * 256 + 128 * half);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) afr[mt][ks] = __builtin_bit_cast(bf16x8, p[ks]);
    } else {
      const int64_t qr = (int64_t)row * 64 + head;
      const u32x4* p = reinterpret_cast<const u32x4*>(qI + qr * 64 + 32 * half);
      const u32x4 w0 = p[0], w1 = p[1];
      const float s0 = exp2i((int)qI_scale[qr * 4 + 2 * half] - 127);
      const float s1 = exp2i((int)qI_scale[qr * 4 + 2 * half + 1] - 127);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) afr[mt][ks] = e2m1x8_to_bf16(w0[ks], s0);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) afr[mt][4 + ks] = e2m1x8_to_bf16(w1[ks], s1);
    }
  }
  // weights of the head rows this lane's accumulators hold:
  // register r of tile mt is head 32*mt + 8*(r/4) + 4*half + r%4
  float wr[2][16];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      wr[mt][r] = w[(int64_t)row * 64 + 32 * mt + 8 * (r >> 2) + 4 * half + (r & 3)];

  // raw key bytes of one 32-entry sub-tile (bf16: 128 B per lane; MXFP4: 32 B
  // of codes + the row's 4 scale bytes), prefetched one sub-tile ahead
  struct Raw {
    u32x4 v[MX ? 2 : 8];
    uint32_t sc;
  };
  auto fetch = [&](int base, Raw& r) {
    const int n = base + col;
    const int64_t kr = (int64_t)b * Nmax + (n < e1 ? n : e0);
    if (!MX) {
      const u32x4* p = reinterpret_cast<const u32x4*>(kI + kr * 256 + 128 * half);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) r.v[ks] = p[ks];
      r.sc = 0;
    } else {
      const u32x4* p = reinterpret_cast<const u32x4*>(kI + kr * 64 + 32 * half);
      r.v[0] = p[0];
      r.v[1] = p[1];
      r.sc = *reinterpret_cast<const uint32_t*>(kI_scale + kr * 4);
    }
  };
  constexpr int STEP = IDX_WAVES * IDX_SUB;
  Raw cur, nxt;
  int base = e0 + wave * IDX_SUB;
  if (base < e1) fetch(base, cur);
  for (; base < e1; base += STEP) {
    if (base + STEP < e1) fetch(base + STEP, nxt);
    bf16x8 bfr[8];
    if (!MX) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) bfr[ks] = __builtin_bit_cast(bf16x8, cur.v[ks]);
    } else {
      const float s0 = exp2i((int)((cur.sc >> (16 * half)) & 0xFFu) - 127);
      const float s1 = exp2i((int)((cur.sc >> (16 * half + 8)) & 0xFFu) - 127);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) bfr[ks] = e2m1x8_to_bf16(cur.v[0][ks], s0);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) bfr[4 + ks] = e2m1x8_to_bf16(cur.v[1][ks], s1);
    }
    f32x16 acc0 = {}, acc1 = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr[0][ks], bfr[ks], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr[1][ks], bfr[ks], acc1, 0, 0, 0);
    }
    float sc = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sc = fmaf(wr[0][r], fmaxf(acc0[r], 0.f), sc);
      sc = fmaf(wr[1][r], fmaxf(acc1[r], 0.f), sc);
    }
    sc += __shfl_xor(sc, 32);
    const int n = base + col;
    if (half == 0 && n < e1) {
      const int64_t o = (int64_t)row * Nmax + n;
      if (score_bf16)
        reinterpret_cast<uint16_t*>(scores)[o] = (uint16_t)f32_to_bf16(sc);
      else
        reinterpret_cast<float*>(scores)[o] = sc;
    }
    cur = nxt;
  }
}

hipError_t launch_indexer(const void* qI, const uint8_t* qI_scale, csa_dtype in_t, const float* w,
                          const void* kI, const uint8_t* kI_scale, const int32_t* q_pos,
                          const int32_t* n_entries, int B, int Tq, int nI, int cI, int Nmax,
                          int m, void* scores, csa_dtype score_t, hipStream_t s) {
  const int rows = B * Tq;
  if (rows == 0 || Nmax == 0) return hipSuccess;
  const int sbf = score_t == CSA_BF16;
  if ((in_t == CSA_BF16 || in_t == CSA_MXFP4) && nI == 64 && cI == 128) {
    // about three blocks per CU over the whole call; a block covers a
    // multiple of 128 entries (4 waves x 32)
    const int64_t want = ((int64_t)Nmax * rows + 767) / 768;
    int epb = (int)(((want + 127) / 128) * 128);
    epb = epb < 256 ? 256 : (epb > 8192 ? 8192 : epb);
    dim3 grid((unsigned)(((int64_t)Nmax + epb - 1) / epb * rows));
    if (in_t == CSA_BF16)
      hipLaunchKernelGGL(indexer_mfma_kernel<false>, grid, dim3(IDX_WAVES * 64), 0, s,
                         (const uint8_t*)qI, qI_scale, w, (const uint8_t*)kI, kI_scale, q_pos,
                         n_entries, Tq, Nmax, m, epb, scores, sbf);
    else
      hipLaunchKernelGGL(indexer_mfma_kernel<true>, grid, dim3(IDX_WAVES * 64), 0, s,
                         (const uint8_t*)qI, qI_scale, w, (const uint8_t*)kI, kI_scale, q_pos,
                         n_entries, Tq, Nmax, m, epb, scores, sbf);
  } else {
    dim3 grid((unsigned)(((int64_t)Nmax + 255) / 256 * rows));
    const size_t shm = (size_t)(nI * cI + nI) * sizeof(float);
    hipLaunchKernelGGL(indexer_generic_kernel, grid, dim3(256), shm, s, (const uint8_t*)qI,
                       qI_scale, in_t, w, (const uint8_t*)kI, kI_scale, q_pos, n_entries, Tq, nI,
                       cI, Nmax, m, scores, sbf);
  }
  return hipGetLastError();
}

}  // namespace csa
