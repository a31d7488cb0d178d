// Block-scaled FP8 GEMM for gfx950 with a 3-slot LDS ring fed by
// buffer-to-LDS loads: the kernel for large dense problems, the M-grouped
// contiguous form, and the M-grouped masked form (one 256-row tile covers
// an expert's whole capacity, so each expert's weights stream once; 16-row
// MFMA tiles past masked_m are skipped).
//
// The computation is the one of Lesson 13 (hpc.payai.win), Fig. 13-1 and its
// closed-form equation: for every 128-wide K block the fp8 partial product of
// a tile is formed by the matrix cores and promoted into an fp32 accumulator
// with alpha[row, k] * beta[k]; the epilogue rounds to bf16.
//
// Organisation:
//   * 512 threads = 8 wave64s (two per SIMD), arranged WGM x WGN, each wave a
//     64 x 64 sub-tile of 4 x 4 v_mfma_f32_16x16x128_f8f6f4 tiles; one MFMA
//     covers a whole 128-deep K block;
//   * A, B and the row scales alpha of K block k travel HBM -> LDS with
//     gfx950 buffer-to-LDS loads (no staging registers) into ring slot k % 3,
//     issued three K blocks ahead: a wave first copies all its operands of
//     block k from LDS into registers, so after one s_barrier per K block
//     slot k % 3 is free again and receives block k+3 while the MFMAs run
//     from registers.  Each wave waits for its own loads with an explicit
//     vmcnt; the three slots are separate LDS arrays so the compiler can tell
//     in-flight DMA targets from the slot being read;
//   * LDS rows are 128 bytes; 16-byte chunk c of row r is stored at chunk
//     c ^ (r % 8), so 8 consecutive rows read at one logical chunk hit 8
//     distinct 16-byte bank groups (conflict-free at 128 B/clk);
//   * a lane's MFMA operand is row (lane % 16), K chunks q and q + 4
//     (q = lane / 16) of the 128-byte block -- the same K permutation for A
//     and B, so every dot product is unchanged.  B is the row operand and A
//     the column operand; B rows enter LDS in a permuted order so that each
//     lane ends with 16 consecutive output columns of one row (32-byte
//     stores) and one row scale per row tile;
//   * promotion: each 16x16x128 MFMA writes a fresh fp32 partial of one
//     128-K block, and one FMA per element adds it into the fp32
//     accumulator with that block's alpha[row] * beta (exact for any scale,
//     zero included; measured as fast here as folding the scales into a
//     rescaled accumulator, since the other wave of the SIMD fills the
//     MFMA -> FMA latency);
//   * tiles are mapped so each XCD runs a contiguous, m-grouped range
//     (operand reuse in that XCD's L2).

#include "dg_internal.hpp"
#include "gemm_common.hpp"

namespace dg {
namespace {

constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) buffer, gfx9 family

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, kRsrcWord3);
}

template <int WGM, int WGN, int MODE>
__global__ void __launch_bounds__(512) fp8_gemm_lds_kernel(GemmParams p) {
  // The body uses device-only builtins (buffer resources); the host pass only
  // needs the kernel's signature to emit its launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int TM = 4;
  constexpr int TN = 4;
  constexpr int BM = WGM * 64;
  constexpr int BN = WGN * 64;
  constexpr int NWAVES = 8;
  constexpr int A_INS = BM / 8 / NWAVES;  // 1 KB (8-row) loads per wave per K block
  constexpr int B_INS = BN / 8 / NWAVES;
  constexpr int L_BLOCK = A_INS + B_INS + 1;  // + one alpha load per wave
  constexpr int GM = 4;                      // m-tiles per tile group
  static_assert(WGM * WGN == NWAVES, "eight waves");
  static_assert(BM % 64 == 0 && BN % 64 == 0 && A_INS >= 1 && B_INS >= 1, "tile");
  static_assert(BM <= 256, "alpha slots");
  static_assert(L_BLOCK < 64, "vmcnt range");

  __shared__ __attribute__((aligned(1024))) uint8_t sA0[BM * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t sA1[BM * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t sA2[BM * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[BN * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t sB1[BN * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t sB2[BN * 128];
  // alpha: 64 rows per wave; waves past BM/64 load clamped rows nobody reads
  __shared__ __attribute__((aligned(256))) float sS0[NWAVES * 64];
  __shared__ __attribute__((aligned(256))) float sS1[NWAVES * 64];
  __shared__ __attribute__((aligned(256))) float sS2[NWAVES * 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN;
  const int wn = wave % WGN;

  int mt, nt, grp = 0;
  if (MODE == kMasked) {
    // (expert, m-tile, n-tile), n fastest: an expert's tiles are adjacent, so
    // each XCD streams a few experts' weights and reuses their activations
    const int t = xcd_tile(blockIdx.x, p.G * p.m_tiles * p.n_tiles);
    const int per = p.m_tiles * p.n_tiles;
    grp = t / per;
    mt = (t - grp * per) / p.n_tiles;
    nt = t - grp * per - mt * p.n_tiles;
  } else {
    grouped_mn(xcd_tile(blockIdx.x, p.m_tiles * p.n_tiles), p.m_tiles, p.n_tiles, GM, &mt, &nt);
  }

  const int K = p.K;
  const int N = p.N;
  const int KB = K >> 7;
  const int NB = (N + 127) >> 7;
  const int rows = (int)p.rows;
  const int m0 = mt * BM;
  const int n0 = nt * BN;
  const uint8_t* Ap = p.A;
  const float* sfa = p.sfa;
  const uint8_t* Bp = p.B;
  const float* sfb = p.sfb;
  uint16_t* D = p.D;
  int row_limit = rows - m0 < BM ? rows - m0 : BM;
  int expert = 0;

  if (MODE == kMasked) {
    int mm = p.index[grp];
    mm = mm < 0 ? 0 : (mm > rows ? rows : mm);
    if (m0 >= mm) return;  // whole tile past this expert's valid rows (uniform)
    row_limit = mm - m0 < BM ? mm - m0 : BM;
    Ap += (int64_t)grp * rows * K;
    sfa += (int64_t)grp * KB * rows;
    Bp += (int64_t)grp * N * K;
    sfb += (int64_t)grp * NB * KB;
    D += (int64_t)grp * rows * N;
  }

  if (MODE == kContiguous) {
    // expert of this tile = largest valid index among its rows (computed by
    // every wave; rows of an aligned block belong to one expert)
    int e = -1;
    for (int r = lane; r < row_limit; r += 64) {
      const int v = p.index[m0 + r];
      if (v >= 0 && v < p.G) e = v > e ? v : e;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const int o = __shfl_xor(e, off);
      e = o > e ? o : e;
    }
    expert = __builtin_amdgcn_readfirstlane(e);
    if (expert < 0) return;  // padding-only tile (uniform over the workgroup)
    Bp += (int64_t)expert * N * K;
    sfb += (int64_t)expert * NB * KB;
  }

  // masked: A rows past masked_m lie outside the buffer range, so their loads
  // return zeros without touching memory
  const uint32_t a_rows = MODE == kMasked ? (uint32_t)(m0 + row_limit) : (uint32_t)rows;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ap, a_rows * (uint32_t)K);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bp, (uint32_t)N * (uint32_t)K);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(sfa, (uint32_t)rows * (uint32_t)KB * 4u);

  // DMA sources: instruction i of this wave fills LDS rows 8*(i*8 + wave) + lane/8;
  // lane chunk (lane % 8) of row r holds K chunk (lane % 8) ^ (r % 8).  The
  // offsets are linear in i (stride 64 rows); rows past the end of a buffer
  // fall outside its buffer range and read as zeros -- they only feed
  // accumulator rows / columns that are never stored.
  const int dma_chunk = ((lane & 7) ^ ((lane >> 3) & 7)) << 4;
  const uint32_t a_src = (uint32_t)(m0 + 8 * wave + (lane >> 3)) * (uint32_t)K + (uint32_t)dma_chunk;
  // B rows enter LDS permuted: row 16 j + i of a wave's 64-row block holds
  // weight row (i / 4) * 16 + 4 j + i % 4 of it, so that in the MFMA output
  // (B as row operand) lane l holds 16 consecutive columns q * 16 + [0, 16)
  // of one output row.  Instruction i of this wave fills LDS rows
  // 64 i + 8 wave + lane / 8, i.e. local row 8 wave + lane / 8 of block i.
  const int b_loc = 8 * wave + (lane >> 3);
  const int b_perm = ((b_loc & 15) >> 2) * 16 + 4 * (b_loc >> 4) + (b_loc & 3);
  const uint32_t b_src = (uint32_t)(n0 + b_perm) * (uint32_t)K + (uint32_t)dma_chunk;
  const uint32_t dma_stride = 64u * (uint32_t)K;
  const uint32_t s_src = (uint32_t)(m0 + wave * 64 + lane) * 4u;

  // fragment reads: row base + 16 t + (lane % 16), K chunks q and q + 4
  const int q = lane >> 4;
  const uint32_t fr_lo = (uint32_t)((lane & 15) * 128 + ((q ^ (lane & 7)) << 4));
  const uint32_t fr_hi = (uint32_t)((lane & 15) * 128 + (((q + 4) ^ (lane & 7)) << 4));
  const uint32_t a_row0 = (uint32_t)(wm * 64 * 128);
  const uint32_t b_row0 = (uint32_t)(wn * 64 * 128);

  // this wave's weight-scale row (its 64 columns lie in one 128-column block);
  // made explicitly uniform so the per-block read is a scalar load
  int nblk = (n0 + wn * 64) >> 7;
  nblk = nblk < NB ? nblk : NB - 1;
  const DG_CONST float* sfb_w;
  {
    const uint64_t a = reinterpret_cast<uint64_t>(sfb + nblk * KB);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    sfb_w = (const DG_CONST float*)(((uint64_t)hi << 32) | lo);
  }

  // 16-row MFMA tiles of this wave that hold rows to be stored (all four
  // except in the last rows of a grouped problem); the others skip their MFMAs
  int act = (row_limit - wm * 64 + 15) >> 4;
  act = act < 0 ? 0 : (act > TM ? TM : act);
  act = __builtin_amdgcn_readfirstlane(act);

  f32x4 u[TM][TN];  // fp32 accumulators
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) u[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#define DG_SA(st) ((st) == 0 ? sA0 : ((st) == 1 ? sA1 : sA2))
#define DG_SB(st) ((st) == 0 ? sB0 : ((st) == 1 ? sB1 : sB2))
#define DG_SS(st) ((st) == 0 ? sS0 : ((st) == 1 ? sS1 : sS2))

  // all loads of K block kb_ into ring slot st_
#define DG_ISSUE(st_, kb_)                                                                                 \
  do {                                                                                                     \
    const int ks_ = (kb_) << 7;                                                                            \
    _Pragma("unroll") for (int i_ = 0; i_ < A_INS; ++i_)                                                   \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (DG_LDS void*)(DG_SA(st_) + (i_ * NWAVES + wave) * 1024), \
                                                 16, a_src + i_ * dma_stride, ks_, 0, 0);                  \
    _Pragma("unroll") for (int i_ = 0; i_ < B_INS; ++i_)                                                   \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (DG_LDS void*)(DG_SB(st_) + (i_ * NWAVES + wave) * 1024), \
                                                 16, b_src + i_ * dma_stride, ks_, 0, 0);                  \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (DG_LDS void*)(DG_SS(st_) + wave * 64), 4, s_src,         \
                                             (kb_) * rows * 4, 0, 0);                                      \
  } while (0)

#define DG_FRAG(dst_, base_, off_)                                                                         \
  do {                                                                                                     \
    const uint4 lo_ = *reinterpret_cast<const uint4*>((base_) + fr_lo + (off_));                          \
    const uint4 hi_ = *reinterpret_cast<const uint4*>((base_) + fr_hi + (off_));                          \
    dst_ = i32x8{(int)lo_.x, (int)lo_.y, (int)lo_.z, (int)lo_.w, (int)hi_.x, (int)hi_.y, (int)hi_.z, (int)hi_.w}; \
  } while (0)

  // One K block k, its data already in ring slot k % 3:
  //   1. read all of this wave's fragments and row scales of block k into
  //      registers;
  //   2. wait until this wave's loads of block k+1 have landed (only block
  //      k+2's L_BLOCK loads may remain in flight) and its LDS reads of
  //      block k have returned, then one s_barrier: after it block k+1 is
  //      complete in LDS and no wave reads slot k % 3 again;
  //   3. issue block k+3 into slot k % 3 (three blocks of load latency cover);
  //   4. MFMAs and promotion from registers, overlapping the loads in flight.
  // Past the last block the issue repeats the last block into a slot nobody
  // reads again, which keeps the wait count the same in every block.
#define DG_STEP(st_, k_)                                                                                   \
  do {                                                                                                     \
    const float beta_ = sfb_w[(k_)];                                                                       \
    const uint8_t* as_ = DG_SA(st_) + a_row0;                                                              \
    const uint8_t* bs_ = DG_SB(st_) + b_row0;                                                              \
    i32x8 af_[TM];                                                                                         \
    i32x8 bf_[TN];                                                                                         \
    float al_[TM];                                                                                         \
    _Pragma("unroll") for (int i_ = 0; i_ < TM; ++i_) {                                                    \
      DG_FRAG(af_[i_], as_, i_ * 2048);                                                                    \
      al_[i_] = DG_SS(st_)[wm * 64 + i_ * 16 + (lane & 15)];                                               \
    }                                                                                                      \
    _Pragma("unroll") for (int j_ = 0; j_ < TN; ++j_) DG_FRAG(bf_[j_], bs_, j_ * 2048);                   \
    wait_vmcnt<L_BLOCK>();                                                                                 \
    wait_lgkmcnt0(); /* own reads of slot k done before anyone may refill it */                           \
    __builtin_amdgcn_s_barrier();                                                                          \
    DG_ISSUE((st_), (k_) + 3 < KB ? (k_) + 3 : KB - 1);                                                   \
    float sc_[TM];                                                                                         \
    _Pragma("unroll") for (int i_ = 0; i_ < TM; ++i_) sc_[i_] = al_[i_] * beta_;                           \
    _Pragma("unroll") for (int j_ = 0; j_ < TN; ++j_) {                                                    \
      _Pragma("unroll") for (int i_ = 0; i_ < TM; ++i_) {                                                  \
        if (MODE != kMasked || i_ < act) {                                                                 \
          const f32x4 t_ = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf_[j_], af_[i_], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0); \
          _Pragma("unroll") for (int v_ = 0; v_ < 4; ++v_) u[i_][j_][v_] = __builtin_fmaf(t_[v_], sc_[i_], u[i_][j_][v_]); \
        }                                                                                                  \
      }                                                                                                    \
    }                                                                                                      \
  } while (0)

  DG_ISSUE(0, 0);
  DG_ISSUE(1, 1 < KB ? 1 : KB - 1);
  DG_ISSUE(2, 2 < KB ? 2 : KB - 1);
  wait_vmcnt<2 * L_BLOCK>();  // block 0 landed (this wave's part)
  __builtin_amdgcn_s_barrier();
  int k = 0;
  for (; k + 3 <= KB; k += 3) {
    DG_STEP(0, k);
    DG_STEP(1, k + 1);
    DG_STEP(2, k + 2);
  }
  if (k < KB) DG_STEP(0, k);
  if (k + 1 < KB) DG_STEP(1, k + 1);
  wait_vmcnt<0>();  // no LDS writes may be in flight when the workgroup ends

#undef DG_STEP
#undef DG_FRAG
#undef DG_ISSUE
#undef DG_SA
#undef DG_SB
#undef DG_SS

  // epilogue: for row tile i, lane l holds output row wm*64 + 16 i + l % 16
  // and its 16 consecutive columns wn*64 + q*16 + 4 j + v: two 16-byte
  // stores.  N is a multiple of 16, so a lane's columns are all inside N or
  // all outside.
  const int gc0 = n0 + wn * 64 + q * 16;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int r = wm * 64 + i * 16 + (lane & 15);
    if (r >= row_limit || gc0 >= N) continue;
    const int64_t gr = (int64_t)m0 + r;
    if (MODE == kContiguous && p.index[gr] != expert) continue;
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      w[2 * j] = pack_bf16x2(u[i][j][0], u[i][j][1]);
      w[2 * j + 1] = pack_bf16x2(u[i][j][2], u[i][j][3]);
    }
    uint4* dst = reinterpret_cast<uint4*>(D + gr * N + gc0);
    dst[0] = uint4{w[0], w[1], w[2], w[3]};
    dst[1] = uint4{w[4], w[5], w[6], w[7]};
  }
#endif  // __HIP_DEVICE_COMPILE__
}

template <int WGM, int WGN>
hipError_t launch_lds_cfg(int mode, const GemmParams& p, hipStream_t stream) {
  const int64_t grid = (int64_t)p.m_tiles * p.n_tiles * (mode == kMasked ? p.G : 1);
  if (grid <= 0) return hipSuccess;
  if (mode == kContiguous)
    hipLaunchKernelGGL((fp8_gemm_lds_kernel<WGM, WGN, kContiguous>), dim3((unsigned)grid), dim3(512), 0, stream, p);
  else if (mode == kMasked)
    hipLaunchKernelGGL((fp8_gemm_lds_kernel<WGM, WGN, kMasked>), dim3((unsigned)grid), dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((fp8_gemm_lds_kernel<WGM, WGN, kDense>), dim3((unsigned)grid), dim3(512), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

TileShape lds_tile_shape(int cfg) { return cfg == kLds256x128 ? TileShape{256, 128} : TileShape{128, 256}; }

hipError_t launch_gemm_lds(int mode, int cfg, const GemmParams& p, hipStream_t stream) {
  return cfg == kLds256x128 ? launch_lds_cfg<4, 2>(mode, p, stream) : launch_lds_cfg<2, 4>(mode, p, stream);
}

}  // namespace dg
