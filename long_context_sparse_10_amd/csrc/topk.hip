// Top-k selection over the visible index scores (Evidence Ledger Eqs 13-17:
// the top-k scores pick the compressed blocks the core attention reads).
//
// One block per query row.  Scores map to order-preserving unsigned keys; an
// MSB-first radix select with 8-bit digits and LDS histograms finds the k-th
// largest key K*; a stable block-wide compaction in entry order then emits
// every entry with key > K* and the lowest-index entries with key == K* until
// k are taken.  The output is therefore ascending, ties go to the lower index,
// and -1 pads rows with fewer than k visible entries.
#include "common.hpp"
#include "internal.hpp"

namespace csa {

// larger score -> larger key; -0.0 and +0.0 map to neighbouring keys, NaN never occurs
__device__ __forceinline__ uint32_t f32_key(uint32_t u) {
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint32_t bf16_key(uint32_t u) {
  return (u & 0x8000u) ? (~u & 0xFFFFu) : (u | 0x8000u);
}

template <bool BF16>
__device__ __forceinline__ uint32_t load_key(const void* scores, int64_t i) {
  if (BF16) return bf16_key(reinterpret_cast<const uint16_t*>(scores)[i]);
  return f32_key(reinterpret_cast<const uint32_t*>(scores)[i]);
}

// inclusive block scan of one int per thread; returns the inclusive value and
// writes the block total to *total; `ws` is LDS of >= 16 ints
__device__ __forceinline__ int block_scan_incl(int v, int* ws, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  if (lane == 63) ws[wave] = v;
  __syncthreads();
  int pre = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    const int x = ws[i];
    pre += (i < wave) ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return v + pre;
}

template <bool BF16>
__global__ __launch_bounds__(1024) void topk_kernel(const void* __restrict__ scores,
                                                    const int32_t* __restrict__ q_pos,
                                                    const int32_t* __restrict__ n_entries, int Tq,
                                                    int Nmax, int m, int k,
                                                    int32_t* __restrict__ idx) {
  __shared__ int hist[256];
  __shared__ int scan_ws[16];
  __shared__ uint32_t sh_digit;
  __shared__ int sh_above;
  const int row = blockIdx.x, b = row / Tq;
  const int tid = threadIdx.x, nt = blockDim.x;
  const int nv = min(min(n_entries[b], Nmax), (q_pos[row] + 1) / m);
  int32_t* out = idx + (int64_t)row * k;
  const void* srow = BF16 ? (const void*)((const uint16_t*)scores + (int64_t)row * Nmax)
                          : (const void*)((const uint32_t*)scores + (int64_t)row * Nmax);
  if (nv <= k) {
    for (int i = tid; i < k; i += nt) out[i] = i < nv ? i : -1;
    return;
  }
  // ---- radix select of the k-th largest key
  uint32_t prefix = 0, pmask = 0;
  int remaining = k;  // rank still to locate within the current prefix class
  const int nbits = BF16 ? 16 : 32;
  for (int shift = nbits - 8; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += nt) hist[i] = 0;
    __syncthreads();
    for (int s = tid; s < nv; s += nt) {
      const uint32_t key = load_key<BF16>(srow, s);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l owns digits 255-4l .. 252-4l (descending); find the digit where
      // the count of keys with a larger-or-equal digit first reaches `remaining`
      const int d0 = 255 - 4 * tid;
      const int c0 = hist[d0], c1 = hist[d0 - 1], c2 = hist[d0 - 2], c3 = hist[d0 - 3];
      int incl = c0 + c1 + c2 + c3;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (tid >= o) incl += t;
      }
      const int excl = incl - (c0 + c1 + c2 + c3);
      if (excl < remaining && incl >= remaining) {
        int above = excl;
        int d = d0;
        const int cs[4] = {c0, c1, c2, c3};
        for (int q = 0; q < 4; ++q) {
          if (above + cs[q] >= remaining) { d = d0 - q; break; }
          above += cs[q];
        }
        sh_digit = (uint32_t)d;
        sh_above = above;
      }
    }
    __syncthreads();
    remaining -= sh_above;
    prefix |= sh_digit << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t kstar = prefix;
  const int need_eq = remaining;  // entries equal to K* to take, lowest index first
  // ---- stable compaction in entry order
  int run_gt = 0, run_eq = 0;
  for (int base = 0; base < nv; base += nt) {
    const int s = base + tid;
    uint32_t key = 0;
    if (s < nv) key = load_key<BF16>(srow, s);
    const int gt = (s < nv) && key > kstar;
    const int eq = (s < nv) && key == kstar;
    int total;
    const int incl = block_scan_incl(gt | (eq << 16), scan_ws, &total);
    const int excl = incl - (gt | (eq << 16));
    const int gt_before = run_gt + (excl & 0xFFFF), eq_before = run_eq + (excl >> 16);
    const int pos = gt_before + min(eq_before, need_eq);
    if ((gt || (eq && eq_before < need_eq)) && pos < k) out[pos] = s;
    run_gt += total & 0xFFFF;
    run_eq += total >> 16;
  }
}

hipError_t launch_topk(const void* scores, csa_dtype score_t, const int32_t* q_pos,
                       const int32_t* n_entries, int B, int Tq, int Nmax, int m, int k,
                       int32_t* idx, hipStream_t s) {
  const int rows = B * Tq;
  if (rows == 0) return hipSuccess;
  const int threads = Nmax >= 8192 ? 1024 : (Nmax >= 2048 ? 512 : 256);
  if (score_t == CSA_BF16)
    hipLaunchKernelGGL(topk_kernel<true>, dim3(rows), dim3(threads), 0, s, scores, q_pos,
                       n_entries, Tq, Nmax, m, k, idx);
  else
    hipLaunchKernelGGL(topk_kernel<false>, dim3(rows), dim3(threads), 0, s, scores, q_pos,
                       n_entries, Tq, Nmax, m, k, idx);
  return hipGetLastError();
}

}  // namespace csa
