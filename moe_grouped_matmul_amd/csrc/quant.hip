// Fine-grained FP8 quantisers for gfx950.
//
// Lesson 13 "DeepSeek DeepGEMM core architecture and Hopper FP8 operator
// breakdown" (hpc.payai.win), Fig. 13-1: activations get one fp32 scale per
// token per 128 K elements, weights one per 128x128 block; the scale is the
// group's largest magnitude divided by 448, the e4m3 maximum.  The pages leave
// the rounding open; these kernels use IEEE fp32 division for the scale and
// for x / scale, and round-to-nearest-even onto the e4m3 grid (subnormals
// included, ties to even mantissa, sign of zero kept, saturation at 448), so
// the output bytes are unique.  An all-zero group gets scale 1.
//
// UE8M0 variants (newer library versions accept power-of-two scales: Lesson
// 13, the notes after Fig. 13-1; the deep-dive blog, section 3, packs four of
// them into one 32-bit word): the scale is the smallest power of two not
// below amax / 448, stored as its biased exponent byte (2^(c - 127)), and the
// element is scaled by the exact inverse power before the same e4m3
// rounding.  Codes are packed four per int32 along K (block 4w + j in byte
// j, unused bytes zero).
//
// Both kernels are HBM-bound: 4 bytes read and 1 byte (+4 bytes per group)
// written per element.

#include "dg_internal.hpp"

namespace dg {
namespace {

constexpr float kE4M3Max = 448.0f;

// fp32 -> OCP e4m3 (E4M3FN) byte, round to nearest even, saturating.
__device__ __forceinline__ uint32_t e4m3_rne(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t s = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return s | 0x7fu;  // NaN
  if (a >= 0x43e00000u) return s | 0x7eu;  // |y| >= 448 (and inf): saturate
  if (a >= 0x3c800000u) {
    // |y| >= 2^-6: normal e4m3.  Drop 20 of the 23 fp32 mantissa bits with
    // round-to-nearest-even (a carry moves into the exponent by itself), then
    // rebias the exponent from 127 to 7.
    const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
    return s | (r - (120u << 3));
  }
  // Subnormal e4m3: multiples of 2^-9.  |y| * 512 is exact; rint is RNE.
  return s | (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
}

__device__ __forceinline__ float scale_from_amax(float amax) {
  const float s = amax / kE4M3Max;  // IEEE-correct division (no fast-math)
  return s == 0.0f ? 1.0f : s;
}

__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d, float s) {
  return e4m3_rne(a / s) | (e4m3_rne(b / s) << 8) | (e4m3_rne(c / s) << 16) | (e4m3_rne(d / s) << 24);
}

// UE8M0 code of a group: c = 127 + min{e : 448 * 2^e >= amax}, clamped to
// [0, 254]; an all-zero group gets 127.  With amax = 1.f * 2^(E - 127) and
// 448 = 1.75 * 2^8 the minimum is E - 135 when 1.f <= 1.75 (mantissa field
// <= 0x600000) and E - 134 above; subnormal and tiny amax clamp to 0.
__device__ __forceinline__ int ue8m0_code(float amax) {
  const uint32_t u = __float_as_uint(amax);
  if (u == 0) return 127;
  const int c = (int)(u >> 23) - 8 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);
  return (u >> 23) == 0 ? 0 : (c < 0 ? 0 : (c > 254 ? 254 : c));
}

// x * 2^(127 - c): an exact power-of-two scaling (one rounding only when the
// product is an fp32 subnormal, far below the e4m3 grid)
__device__ __forceinline__ uint32_t pack4_pow2(float a, float b, float c, float d, float inv) {
  return e4m3_rne(a * inv) | (e4m3_rne(b * inv) << 8) | (e4m3_rne(c * inv) << 16) | (e4m3_rne(d * inv) << 24);
}

// stores code c of K block kb into its packed word (byte kb % 4); the last
// block of a row also zeroes the word's unused bytes
__device__ __forceinline__ void store_code(uint8_t* word, int kb, int KB, int c) {
  word[kb & 3] = (uint8_t)c;
  if (kb == KB - 1)
    for (int j = (kb & 3) + 1; j < 4; ++j) word[j] = 0;
}

// 1x128 groups: 16 lanes per group, 8 elements per lane (two 16-byte loads).
template <bool UE8M0>
__global__ void __launch_bounds__(256) quant_1x128_kernel(const float* __restrict__ x, uint8_t* __restrict__ q,
                                                          void* __restrict__ sfa, int64_t M, int K,
                                                          int64_t total_groups) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t grp_raw = t >> 4;
  const int sub = threadIdx.x & 15;
  const bool active = grp_raw < total_groups;
  const int64_t grp = active ? grp_raw : total_groups - 1;
  const int KB = K >> 7;
  const int64_t row = grp / KB;  // flattened (g, m)
  const int kb = (int)(grp - row * KB);
  const float* src = x + row * K + ((int64_t)kb << 7) + (sub << 3);
  const float4 v0 = *reinterpret_cast<const float4*>(src);
  const float4 v1 = *reinterpret_cast<const float4*>(src + 4);
  float amax = fmaxf(fmaxf(fmaxf(fabsf(v0.x), fabsf(v0.y)), fmaxf(fabsf(v0.z), fabsf(v0.w))),
                     fmaxf(fmaxf(fabsf(v1.x), fabsf(v1.y)), fmaxf(fabsf(v1.z), fabsf(v1.w))));
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
  if (!active) return;
  uint2 out;
  const int64_t g = row / M;
  const int64_t m = row - g * M;
  if constexpr (UE8M0) {
    const int c = ue8m0_code(amax);
    const float inv = __builtin_ldexpf(1.0f, 127 - c);
    out.x = pack4_pow2(v0.x, v0.y, v0.z, v0.w, inv);
    out.y = pack4_pow2(v1.x, v1.y, v1.z, v1.w, inv);
    if (sub == 0) {
      const int KW = (KB + 3) >> 2;  // packed [G][KW][M] int32
      store_code(reinterpret_cast<uint8_t*>(static_cast<int32_t*>(sfa) + (g * KW + (kb >> 2)) * M + m), kb, KB, c);
    }
  } else {
    const float s = scale_from_amax(amax);
    out.x = pack4(v0.x, v0.y, v0.z, v0.w, s);
    out.y = pack4(v1.x, v1.y, v1.z, v1.w, s);
    if (sub == 0) static_cast<float*>(sfa)[(g * KB + kb) * M + m] = s;
  }
  *reinterpret_cast<uint2*>(q + row * K + ((int64_t)kb << 7) + (sub << 3)) = out;
}

// 128x128 blocks: one 256-thread workgroup per block; thread t covers rows
// (t >> 4) + 16 i (i < 8) and the 8 columns starting at (t & 15) * 8.
template <bool UE8M0>
__global__ void __launch_bounds__(256) quant_128x128_kernel(const float* __restrict__ x, uint8_t* __restrict__ q,
                                                            void* __restrict__ sfb, int64_t N, int K) {
  __shared__ float s_wave_max[4];
  const int KB = K >> 7;
  const int NB = (int)((N + 127) >> 7);
  const int64_t blk = blockIdx.x;  // (g, nb, kb)
  const int kb = (int)(blk % KB);
  const int64_t gn = blk / KB;
  const int nb = (int)(gn % NB);
  const int64_t g = gn / NB;
  const int tid = threadIdx.x;
  const int col = (tid & 15) << 3;
  const int64_t row0 = (int64_t)nb * 128;
  const float* base = x + (g * N) * K + ((int64_t)kb << 7) + col;

  float4 v[8][2];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = row0 + (tid >> 4) + 16 * i;
    if (r < N) {
      v[i][0] = *reinterpret_cast<const float4*>(base + r * K);
      v[i][1] = *reinterpret_cast<const float4*>(base + r * K + 4);
      amax = fmaxf(amax, fmaxf(fmaxf(fmaxf(fabsf(v[i][0].x), fabsf(v[i][0].y)),
                                     fmaxf(fabsf(v[i][0].z), fabsf(v[i][0].w))),
                               fmaxf(fmaxf(fabsf(v[i][1].x), fabsf(v[i][1].y)),
                                     fmaxf(fabsf(v[i][1].z), fabsf(v[i][1].w)))));
    } else {
      v[i][0] = make_float4(0.f, 0.f, 0.f, 0.f);
      v[i][1] = v[i][0];
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((tid & 63) == 0) s_wave_max[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_wave_max[0], s_wave_max[1]), fmaxf(s_wave_max[2], s_wave_max[3]));
  const float s = scale_from_amax(amax);
  const int c = ue8m0_code(amax);
  const float inv = __builtin_ldexpf(1.0f, 127 - c);
  uint8_t* qbase = q + (g * N) * K + ((int64_t)kb << 7) + col;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = row0 + (tid >> 4) + 16 * i;
    if (r < N) {
      uint2 out;
      if constexpr (UE8M0) {
        out.x = pack4_pow2(v[i][0].x, v[i][0].y, v[i][0].z, v[i][0].w, inv);
        out.y = pack4_pow2(v[i][1].x, v[i][1].y, v[i][1].z, v[i][1].w, inv);
      } else {
        out.x = pack4(v[i][0].x, v[i][0].y, v[i][0].z, v[i][0].w, s);
        out.y = pack4(v[i][1].x, v[i][1].y, v[i][1].z, v[i][1].w, s);
      }
      *reinterpret_cast<uint2*>(qbase + r * K) = out;
    }
  }
  if (tid == 0) {
    if constexpr (UE8M0) {
      const int KW = (KB + 3) >> 2;  // packed [G][NB][KW] int32
      store_code(reinterpret_cast<uint8_t*>(static_cast<int32_t*>(sfb) + (g * NB + nb) * KW + (kb >> 2)), kb, KB, c);
    } else {
      static_cast<float*>(sfb)[(g * NB + nb) * KB + kb] = s;
    }
  }
}

}  // namespace

hipError_t launch_quant_1x128(const float* x, uint8_t* q, void* sfa, int64_t G, int64_t M, int64_t K, bool ue8m0,
                              hipStream_t stream) {
  const int64_t groups = G * M * (K / 128);
  const int64_t blocks = (groups * 16 + 255) / 256;
  if (ue8m0)
    hipLaunchKernelGGL(quant_1x128_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, x, q, sfa, M, (int)K,
                       groups);
  else
    hipLaunchKernelGGL(quant_1x128_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, x, q, sfa, M, (int)K,
                       groups);
  return hipGetLastError();
}

hipError_t launch_quant_128x128(const float* x, uint8_t* q, void* sfb, int64_t G, int64_t N, int64_t K, bool ue8m0,
                                hipStream_t stream) {
  const int64_t blocks = G * ((N + 127) / 128) * (K / 128);
  if (ue8m0)
    hipLaunchKernelGGL(quant_128x128_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, x, q, sfb, N, (int)K);
  else
    hipLaunchKernelGGL(quant_128x128_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, x, q, sfb, N, (int)K);
  return hipGetLastError();
}

}  // namespace dg
