// Block-scaled FP8 GEMM D = A . B^T -> bf16 for gfx950 (CDNA4), with the
// dense, M-grouped contiguous and M-grouped masked forms.
//
// What is computed (Lesson 13 "DeepSeek DeepGEMM core architecture and Hopper
// FP8 operator breakdown", hpc.payai.win, Fig. 13-1 and its closed-form
// equation): for every 128-wide K block g the fp8 partial product of a tile is
// formed by the matrix cores, multiplied by alpha[row, g] * beta[col/128, g]
// and added into an fp32 accumulator held in VGPRs ("promotion"); after the
// last K block the accumulator is rounded to bf16 and stored.  The pages'
// Hopper design (TMA, WGMMA, mbarrier rings) is prior art; this is the gfx950
// version:
//   * 256-thread workgroups (4 wave64s), tile BM x BN, K step 128 = one scale
//     block, so a tile's K loop runs over exactly the promotion blocks;
//   * operands move HBM -> VGPR (16-byte global loads, 8 lanes per 128-byte
//     row segment) -> LDS (double buffered, 16-byte chunks XOR-swizzled per
//     row so both the stores and the MFMA fragment reads are conflict-free);
//   * each wave owns a WM x WN sub-tile of 16x16 MFMA tiles and issues one
//     v_mfma_f32_16x16x128_f8f6f4 per tile per K block (the full 128-deep
//     block in one instruction), fed by two ds_read_b128 per operand row;
//   * promotion is one fp32 FMA per accumulator element per K block, with the
//     scale alpha*beta formed once per row (beta is one scalar per tile since
//     BN divides 128);
//   * epilogue: fp32 -> bf16 round-to-nearest-even, stores predicated per row
//     (grouped forms) and per column.
// Small dense problems split K across workgroups into fp32 partials that a
// second kernel sums in a fixed order (deterministic).

#include "dg_internal.hpp"
#include "gemm_common.hpp"

namespace dg {
namespace {

template <int BM, int BN, int WM, int WN, int MODE>
__global__ void __launch_bounds__(256) fp8_gemm_kernel(GemmParams p) {
  constexpr int WAVES_N = BN / WN;
  constexpr int TM = WM / 16;
  constexpr int TN = WN / 16;
  constexpr int A_LD = BM * 8 / 256;  // 16-byte chunks per thread per stage
  constexpr int B_LD = BN * 8 / 256;
  static_assert((BM / WM) * (BN / WN) == 4, "four waves per workgroup");
  static_assert(A_LD >= 1 && B_LD >= 1 && (BM * 8) % 256 == 0 && (BN * 8) % 256 == 0, "tile loads");
  static_assert(128 % BN == 0 || BN % 128 == 0, "tile columns vs beta blocks");
  static_assert(BN <= 128, "one beta block per tile");
  static_assert(BM <= 256, "alpha staging");

  __shared__ __attribute__((aligned(16))) uint8_t s_a[2][BM * 128];
  __shared__ __attribute__((aligned(16))) uint8_t s_b[2][BN * 128];
  __shared__ __attribute__((aligned(16))) float s_alpha[2][BM];
  __shared__ int s_expert;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;

  int bid = blockIdx.x;
  const int ks = bid % p.splits;
  bid /= p.splits;
  const int nt = bid % p.n_tiles;
  bid /= p.n_tiles;
  const int mt = bid % p.m_tiles;
  const int grp = bid / p.m_tiles;

  const int K = p.K;
  const int N = p.N;
  const int KB = K >> 7;
  const int NB = (N + 127) >> 7;
  const int64_t rows = p.rows;
  const int64_t m0 = (int64_t)mt * BM;
  const int n0 = nt * BN;

  const uint8_t* A = p.A;
  const float* sfa = p.sfa;
  const uint8_t* B = p.B;
  const float* sfb = p.sfb;
  uint16_t* D = p.D;
  int row_limit = (int)(rows - m0 < BM ? rows - m0 : BM);
  int expert = 0;

  if (MODE == kMasked) {
    int mm = p.index[grp];
    mm = mm < 0 ? 0 : (mm > rows ? (int)rows : mm);
    if (m0 >= mm) return;  // whole tile past this expert's valid rows
    row_limit = (int)(mm - m0 < BM ? mm - m0 : BM);
    A += (int64_t)grp * rows * K;
    sfa += (int64_t)grp * KB * rows;
    B += (int64_t)grp * N * K;
    sfb += (int64_t)grp * NB * KB;
    D += (int64_t)grp * rows * N;
  } else if (MODE == kContiguous) {
    if (tid == 0) s_expert = -1;
    __syncthreads();
    if (tid < row_limit) {
      const int e = p.index[m0 + tid];
      if (e >= 0 && e < p.G) atomicMax(&s_expert, e);
    }
    __syncthreads();
    expert = s_expert;
    if (expert < 0) return;  // padding-only tile
    B += (int64_t)expert * N * K;
    sfb += (int64_t)expert * NB * KB;
  }

  const int kb0 = ks * p.kb_per_split;
  const int kb1 = (kb0 + p.kb_per_split < KB) ? kb0 + p.kb_per_split : KB;

  // HBM -> registers for K block kb (Stage::load) and registers -> LDS
  // (Stage::store).  Rows past the buffer end are clamped to the last row:
  // they only feed accumulator rows/columns that are never stored.
  struct Stage {
    uint4 a[A_LD];
    uint4 b[B_LD];
    float alpha;
  };
  Stage st;
  st.alpha = 0.0f;

#define DG_GLOAD(kb_)                                                                                       \
  do {                                                                                                       \
    const int64_t kofs_ = (int64_t)(kb_) << 7;                                                               \
    _Pragma("unroll") for (int i_ = 0; i_ < A_LD; ++i_) {                                                    \
      const int c_ = tid + i_ * 256;                                                                         \
      int64_t gr_ = m0 + (c_ >> 3);                                                                          \
      gr_ = gr_ < rows ? gr_ : rows - 1;                                                                     \
      st.a[i_] = *reinterpret_cast<const uint4*>(A + gr_ * K + kofs_ + ((c_ & 7) << 4));                    \
    }                                                                                                        \
    _Pragma("unroll") for (int i_ = 0; i_ < B_LD; ++i_) {                                                    \
      const int c_ = tid + i_ * 256;                                                                         \
      int gn_ = n0 + (c_ >> 3);                                                                              \
      gn_ = gn_ < N ? gn_ : N - 1;                                                                           \
      st.b[i_] = *reinterpret_cast<const uint4*>(B + (int64_t)gn_ * K + kofs_ + ((c_ & 7) << 4));           \
    }                                                                                                        \
    if (tid < BM) {                                                                                          \
      int64_t gr_ = m0 + tid;                                                                                \
      gr_ = gr_ < rows ? gr_ : rows - 1;                                                                     \
      st.alpha = sfa[(int64_t)(kb_) * rows + gr_];                                                           \
    }                                                                                                        \
  } while (0)

#define DG_LSTORE(buf_)                                                                                      \
  do {                                                                                                       \
    _Pragma("unroll") for (int i_ = 0; i_ < A_LD; ++i_) {                                                    \
      const int c_ = tid + i_ * 256;                                                                         \
      const int r_ = c_ >> 3;                                                                                \
      *reinterpret_cast<uint4*>(&s_a[buf_][r_ * 128 + (((c_ & 7) ^ swz(r_)) << 4)]) = st.a[i_];            \
    }                                                                                                        \
    _Pragma("unroll") for (int i_ = 0; i_ < B_LD; ++i_) {                                                    \
      const int c_ = tid + i_ * 256;                                                                         \
      const int r_ = c_ >> 3;                                                                                \
      *reinterpret_cast<uint4*>(&s_b[buf_][r_ * 128 + (((c_ & 7) ^ swz(r_)) << 4)]) = st.b[i_];            \
    }                                                                                                        \
    if (tid < BM) s_alpha[buf_][tid] = st.alpha;                                                             \
  } while (0)

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const float* sfb_tile = sfb + (int64_t)(n0 >> 7) * KB;
  const int kq = (lane >> 4) * 2;  // this lane's first 16-byte K chunk (32 K values per lane)

  DG_GLOAD(kb0);
  DG_LSTORE(0);
  __syncthreads();

  for (int kb = kb0; kb < kb1; ++kb) {
    const int cur = (kb - kb0) & 1;
    const bool more = kb + 1 < kb1;
    // the last iteration re-loads its own block (in bounds, never stored) so
    // the staging registers have one unconditional definition per iteration
    DG_GLOAD(more ? kb + 1 : kb);
    const float beta = sfb_tile[kb];

    i32x8 fa[TM];
    i32x8 fb[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm * WM + i * 16 + (lane & 15);
      const uint8_t* rowp = &s_a[cur][r * 128];
      const uint4 lo = *reinterpret_cast<const uint4*>(rowp + ((kq ^ swz(r)) << 4));
      const uint4 hi = *reinterpret_cast<const uint4*>(rowp + (((kq + 1) ^ swz(r)) << 4));
      fa[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int r = wn * WN + j * 16 + (lane & 15);
      const uint8_t* rowp = &s_b[cur][r * 128];
      const uint4 lo = *reinterpret_cast<const uint4*>(rowp + ((kq ^ swz(r)) << 4));
      const uint4 hi = *reinterpret_cast<const uint4*>(rowp + (((kq + 1) ^ swz(r)) << 4));
      fb[j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    // promotion scales for this lane's accumulator rows: row = 4 * (lane / 16) + v
    f32x4 sc[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const f32x4 al = *reinterpret_cast<const f32x4*>(&s_alpha[cur][wm * WM + i * 16 + (lane >> 4) * 4]);
      sc[i] = al * beta;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[i], fb[j], zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i][j][v] = __builtin_fmaf(part[v], sc[i][v], acc[i][j][v]);
      }
    }
    if (more) DG_LSTORE(cur ^ 1);
    __syncthreads();
  }

  // Epilogue.  MFMA 16x16 output layout: lane holds column (lane & 15) and
  // rows 4 * (lane >> 4) + v of its tile.
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = wm * WM + i * 16 + (lane >> 4) * 4 + v;
      if (r >= row_limit) continue;
      const int64_t gr = m0 + r;
      if (MODE == kContiguous && p.index[gr] != expert) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int gc = n0 + wn * WN + j * 16 + (lane & 15);
        if (gc >= N) continue;
        if (MODE == kDense && p.splits > 1) {
          p.ws[((int64_t)ks * rows + gr) * N + gc] = acc[i][j][v];
        } else {
          D[gr * N + gc] = f32_to_bf16_rne(acc[i][j][v]);
        }
      }
    }
  }
}

#undef DG_GLOAD
#undef DG_LSTORE

// Sums the split-K partials in split order and rounds to bf16.
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* __restrict__ ws, uint16_t* __restrict__ D,
                                                            int64_t mn, int splits) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= mn) return;
  float4 s = *reinterpret_cast<const float4*>(ws + i);
  for (int k = 1; k < splits; ++k) {
    const float4 t = *reinterpret_cast<const float4*>(ws + (int64_t)k * mn + i);
    s.x += t.x;
    s.y += t.y;
    s.z += t.z;
    s.w += t.w;
  }
  ushort4 o;
  o.x = f32_to_bf16_rne(s.x);
  o.y = f32_to_bf16_rne(s.y);
  o.z = f32_to_bf16_rne(s.z);
  o.w = f32_to_bf16_rne(s.w);
  *reinterpret_cast<ushort4*>(D + i) = o;
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(int mode, const GemmParams& p, int groups, hipStream_t stream) {
  const int64_t grid = (int64_t)groups * p.m_tiles * p.n_tiles * p.splits;
  if (grid <= 0) return hipSuccess;
  switch (mode) {
    case kDense:
      hipLaunchKernelGGL((fp8_gemm_kernel<BM, BN, WM, WN, kDense>), dim3((unsigned)grid), dim3(256), 0, stream, p);
      break;
    case kContiguous:
      hipLaunchKernelGGL((fp8_gemm_kernel<BM, BN, WM, WN, kContiguous>), dim3((unsigned)grid), dim3(256), 0, stream,
                         p);
      break;
    default:
      hipLaunchKernelGGL((fp8_gemm_kernel<BM, BN, WM, WN, kMasked>), dim3((unsigned)grid), dim3(256), 0, stream, p);
      break;
  }
  return hipGetLastError();
}

}  // namespace

TileShape tile_shape(int cfg) {
  switch (cfg) {
    case kTile128x128:
      return {128, 128};
    case kTile64x128:
      return {64, 128};
    default:
      return {64, 64};
  }
}

hipError_t launch_gemm(int mode, int cfg, const GemmParams& p, int groups, hipStream_t stream) {
  hipError_t e;
  switch (cfg) {
    case kTile128x128:
      e = launch_cfg<128, 128, 64, 64>(mode, p, groups, stream);
      break;
    case kTile64x128:
      e = launch_cfg<64, 128, 32, 64>(mode, p, groups, stream);
      break;
    default:
      e = launch_cfg<64, 64, 32, 32>(mode, p, groups, stream);
      break;
  }
  if (e != hipSuccess) return e;
  if (mode == kDense && p.splits > 1) {
    const int64_t mn = p.rows * p.N;
    const int64_t blocks = (mn / 4 + 255) / 256;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p.ws, p.D, mn, p.splits);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace dg
