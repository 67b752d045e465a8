// Top-k selection over the visible index scores (Evidence Ledger Eqs 13-17:
// the top-k scores pick the compressed blocks the core attention reads).
//
// One block per query row.  Scores map to order-preserving unsigned keys.  An
// MSB-first radix select with LDS histograms finds the k-th largest key K*;
// then every entry with key > K* and the lowest-index entries with key == K*
// (until k are taken) are written in ascending entry order, so ties go to the
// lower index, and rows with fewer than k visible entries are padded with -1.
//
// Rows of up to KPT * blockDim entries keep their keys in registers: thread t
// owns the contiguous entries [KPT t, KPT t + KPT), every radix pass works on
// registers, and the ordered compaction needs a single block-wide scan.
// Longer rows stream their keys from memory on every pass.
#include "common.hpp"
#include "internal.hpp"

namespace csa {

// larger score -> larger key; NaN never occurs
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

// exclusive block scan of one int per thread; *total gets the block sum.
// `ws` is LDS of >= 16 ints.  Every thread of the block must call.
__device__ __forceinline__ int block_scan_excl(int v, int* ws, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(x, o);
    if (lane >= o) x += t;
  }
  if (lane == 63) ws[wave] = x;
  __syncthreads();
  int pre = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    const int y = ws[i];
    pre += (i < wave) ? y : 0;
    tot += y;
  }
  __syncthreads();
  *total = tot;
  return x - v + pre;
}

// Locate the digit of the `remaining`-th largest key among the keys counted in
// hist[0..nbins) (descending digits).  Wave 0 scans; the digit and the count of
// keys in larger digits land in *digit / *above.  nbins is a multiple of 64.
__device__ __forceinline__ void find_digit(const int* hist, int nbins, int remaining,
                                           uint32_t* digit, int* above) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  const int per = nbins / 64;
  const int top = nbins - 1 - per * lane;  // this lane scans digits top .. top-per+1
  int cnt = 0;
  for (int i = 0; i < per; ++i) cnt += hist[top - i];
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  const int excl = incl - cnt;
  if (excl < remaining && incl >= remaining) {
    int acc = excl;
    for (int i = 0; i < per; ++i) {
      const int h = hist[top - i];
      if (acc + h >= remaining) {
        *digit = (uint32_t)(top - i);
        *above = acc;
        break;
      }
      acc += h;
    }
  }
}

template <bool BF16, int KPT>
__global__ __launch_bounds__(1024) void topk_kernel(const void* __restrict__ scores,
                                                    const int32_t* __restrict__ q_pos,
                                                    const int32_t* __restrict__ n_entries, int Tq,
                                                    int Nmax, int m, int k,
                                                    int32_t* __restrict__ idx) {
  __shared__ int hist[2048];
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
  constexpr int KR = KPT > 0 ? KPT : 1;
  const bool in_regs = KPT > 0 && nv <= KR * nt;
  // ---- keys in registers: contiguous chunk per thread
  uint32_t key[KR];
  const int s0 = tid * KR;
  if (in_regs) {
#pragma unroll
    for (int i = 0; i < KR; ++i) key[i] = (s0 + i < nv) ? load_key<BF16>(srow, s0 + i) : 0u;
  }
  // ---- radix select: digits of 11/11/10 bits (fp32 keys) or 8/8 bits (bf16 keys)
  uint32_t prefix = 0u, pmask = 0u;
  int remaining = k;  // rank still to locate inside the current prefix class
  int shift = BF16 ? 16 : 32;
  while (shift > 0) {
    const int width = BF16 ? 8 : (shift == 32 || shift == 21 ? 11 : 10);
    shift -= width;
    const int nbins = 1 << width;
    const uint32_t dmask = (uint32_t)nbins - 1u;
    for (int i = tid; i < nbins; i += nt) hist[i] = 0;
    __syncthreads();
    if (in_regs) {
#pragma unroll
      for (int i = 0; i < KR; ++i)
        if (s0 + i < nv && (key[i] & pmask) == prefix)
          atomicAdd(&hist[(key[i] >> shift) & dmask], 1);
    } else {
      for (int s = tid; s < nv; s += nt) {
        const uint32_t kk = load_key<BF16>(srow, s);
        if ((kk & pmask) == prefix) atomicAdd(&hist[(kk >> shift) & dmask], 1);
      }
    }
    __syncthreads();
    find_digit(hist, nbins, remaining, &sh_digit, &sh_above);
    __syncthreads();
    remaining -= sh_above;
    prefix |= sh_digit << shift;
    pmask |= dmask << shift;
  }
  const uint32_t kstar = prefix;
  const int need_eq = remaining;  // entries equal to K* to take, lowest index first
  // ---- ordered compaction
  if (in_regs) {
    int gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < KR; ++i) {
      const bool ok = s0 + i < nv;
      gt += (ok && key[i] > kstar) ? 1 : 0;
      eq += (ok && key[i] == kstar) ? 1 : 0;
    }
    int total;
    const int excl = block_scan_excl(gt | (eq << 16), scan_ws, &total);
    int gt_before = excl & 0xFFFF, eq_before = excl >> 16;
#pragma unroll
    for (int i = 0; i < KR; ++i) {
      const bool ok = s0 + i < nv;
      const bool g = ok && key[i] > kstar, e = ok && key[i] == kstar;
      if (g || (e && eq_before < need_eq)) {
        const int pos = gt_before + min(eq_before, need_eq);
        if (pos < k) out[pos] = s0 + i;
      }
      gt_before += g ? 1 : 0;
      eq_before += e ? 1 : 0;
    }
  } else {
    int run_gt = 0, run_eq = 0;
    for (int base = 0; base < nv; base += nt) {
      const int s = base + tid;
      uint32_t kk = 0;
      if (s < nv) kk = load_key<BF16>(srow, s);
      const int g = (s < nv) && kk > kstar;
      const int e = (s < nv) && kk == kstar;
      int total;
      const int excl = block_scan_excl(g | (e << 16), scan_ws, &total);
      const int gt_before = run_gt + (excl & 0xFFFF), eq_before = run_eq + (excl >> 16);
      const int pos = gt_before + min(eq_before, need_eq);
      if ((g || (e && eq_before < need_eq)) && pos < k) out[pos] = s;
      run_gt += total & 0xFFFF;
      run_eq += total >> 16;
    }
  }
}

hipError_t launch_topk(const void* scores, csa_dtype score_t, const int32_t* q_pos,
                       const int32_t* n_entries, int B, int Tq, int Nmax, int m, int k,
                       int32_t* idx, hipStream_t s) {
  const int rows = B * Tq;
  if (rows == 0) return hipSuccess;
  const int threads = Nmax > 4096 ? 1024 : (Nmax > 1024 ? 256 : 64);
  const int kpt = (Nmax + threads - 1) / threads;
  const bool bf = score_t == CSA_BF16;
#define CSA_TOPK(BF, KP)                                                                   \
  hipLaunchKernelGGL((topk_kernel<BF, KP>), dim3(rows), dim3(threads), 0, s, scores, q_pos, \
                     n_entries, Tq, Nmax, m, k, idx)
  // register-resident rows: per-thread counts stay below 2^16 for the packed scan
  if (kpt <= 16) {
    if (bf) CSA_TOPK(true, 16); else CSA_TOPK(false, 16);
  } else {
    if (bf) CSA_TOPK(true, 0); else CSA_TOPK(false, 0);
  }
#undef CSA_TOPK
  return hipGetLastError();
}

}  // namespace csa
