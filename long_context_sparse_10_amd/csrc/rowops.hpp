// Block-level row finishing shared by the compressor and the row-prep kernel:
// RMSNorm, partial RoPE and encoding into the cache formats.
#pragma once

#include "common.hpp"

namespace csa {

// sum over the whole block; `red` is LDS scratch of at least blockDim/64 floats
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

// The row (c fp32 values) sits in LDS `row`; every thread of the block calls.
// Evidence Ledger Section 2.3.3: RMSNorm of the entry, then RoPE of its last
// d_r channels (adjacent pairs) at `pos`; then the row is stored in out_t.
__device__ void finish_row(float* row, int c, const float* __restrict__ norm_w, float eps,
                           int d_r, const Rope& rt, double pos, uint8_t* __restrict__ out,
                           uint8_t* __restrict__ out_scale, csa_dtype out_t, float* red) {
  const int tid = threadIdx.x, nt = blockDim.x;
  if (norm_w != nullptr) {
    float ss = 0.f;
    for (int j = tid; j < c; j += nt) ss += row[j] * row[j];
    ss = block_sum(ss, red);
    const float inv = 1.0f / sqrtf(ss / (float)c + eps);
    for (int j = tid; j < c; j += nt) row[j] = row[j] * inv * norm_w[j];
    __syncthreads();
  }
  if (d_r > 0) {
    for (int u = tid; u < d_r / 2; u += nt) {
      float cs, sn;
      rope_cs(rt, pos, u, &cs, &sn);
      const int i0 = c - d_r + 2 * u;
      const float a = row[i0], b = row[i0 + 1];
      row[i0] = a * cs - b * sn;
      row[i0 + 1] = a * sn + b * cs;
    }
    __syncthreads();
  }
  switch (out_t) {
    case CSA_F32: {
      float* o = reinterpret_cast<float*>(out);
      for (int j = tid; j < c; j += nt) o[j] = row[j];
      break;
    }
    case CSA_BF16: {
      uint16_t* o = reinterpret_cast<uint16_t*>(out);
      for (int j = tid; j < c; j += nt) o[j] = (uint16_t)f32_to_bf16(row[j]);
      break;
    }
    case CSA_FP8MIX: {
      const int body = c - d_r;
      for (int j = tid; j < body; j += nt) out[j] = (uint8_t)f32_to_e4m3(row[j]);
      uint16_t* o = reinterpret_cast<uint16_t*>(out + body);
      for (int j = tid; j < d_r; j += nt) o[j] = (uint16_t)f32_to_bf16(row[body + j]);
      break;
    }
    case CSA_MXFP4: {
      for (int blk = tid; blk < c / 32; blk += nt) {
        const float* v = row + 32 * blk;
        float amax = 0.f;
        for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
        const int ex = mx_scale_exp(amax);
        const float inv_scale = exp2i(-ex);   // exact power of two (ex >= -127)
        uint32_t words[4];
        for (int wd = 0; wd < 4; ++wd) {
          uint32_t word = 0;
          for (int i = 0; i < 8; ++i)
            word |= f32_to_e2m1(v[8 * wd + i] * inv_scale) << (4 * i);
          words[wd] = word;
        }
        uint32_t* o = reinterpret_cast<uint32_t*>(out + 16 * blk);
        o[0] = words[0]; o[1] = words[1]; o[2] = words[2]; o[3] = words[3];
        out_scale[blk] = (uint8_t)(ex + 127);
      }
      break;
    }
    default: break;  // formats are checked on the host
  }
}

}  // namespace csa
