// Block-scaled FP8 GEMM for gfx950 when M is small (decode, M <= 128, and up
// to 2048 rows where the output has few columns or K is short): the weights
// B dominate the traffic and are streamed from HBM once per row tile,
// through L2.
//
// The computation is the one of Lesson 13 (hpc.payai.win), Fig. 13-1 and its
// closed-form equation: every 128-wide K block's fp8 partial product is
// promoted into an fp32 accumulator with alpha[row, k] * beta[k]; the
// epilogue rounds to bf16.
//
// Organisation:
//   * a workgroup is 4 wave64s (one per SIMD) and owns a BM-row tile of A
//     (BM = 64, or 128 when 64 < M <= 128, so the weights are read once;
//     several row tiles of 64 or 128 rows when 128 < M <= 2048)
//     times BN = 4 * WN columns of B; each wave owns WN columns.  Should
//     there be several row tiles, the workgroups of one column tile and K
//     split get ids 8 apart (the same XCD under round-robin dispatch);
//   * A and the row scales alpha (shared by the four waves) and each wave's
//     own B columns go HBM/L2 -> LDS with gfx950 buffer-to-LDS loads into a
//     P-slot ring, P - 1 K blocks ahead (P = 4 for 64-row tiles, so two
//     workgroups fit one CU and one's barrier wait hides behind the other's
//     loads; 6 or 4 for 128-row tiles; deeper rings are compiled for
//     measurement).  Fragments are read from LDS while the MFMAs run; the slot
//     of block k - 1 is refilled only after the barrier of block k, which
//     every wave reaches after its reads of block k - 1 have returned.  (B
//     could go straight to registers, but the compiler's wait-count tracking
//     of register loads across the ring loop adds waits that drain most of
//     the prefetch; LDS-targeted loads are tracked exactly);
//   * with M <= 64 (one row tile) each weight line is read by exactly one
//     workgroup, and the weight loads carry the non-temporal cache policy
//     (NT = true: 2-13% faster on the decode shapes); where two 64-row tiles
//     share the weights through one L2, or one 128-row tile reads them, the
//     default policy was as fast or faster;
//   * promotion: each 16x16x128 MFMA (B as row operand, A as column operand)
//     writes a fresh fp32 partial that one FMA per element adds into the
//     accumulator with scale alpha * beta.  With UE8M0 scales (four codes
//     per 32-bit word along K, as in the other kernels) the matrix cores
//     apply beta's code to B and each row's alpha code to A, which is exact
//     for powers of two, and accumulate into the fp32 accumulator (the
//     promotion, bit for bit the separate add of the scaled product);
//   * K is split over several workgroups when the tiles alone cannot occupy
//     the GPU.  Each split stores its fp32 partial tile in the workspace in
//     MFMA fragment order (16-byte stores, coherent across XCDs); the last
//     split of a tile to finish (agent-scope counter) has every wave read
//     back its own fragments of all splits, sums them in split order 0, 1, 2,
//     ... and writes bf16, then resets the counter to zero.  The result is
//     therefore independent of the order in which splits finish.

#include "dg_internal.hpp"
#include "gemm_common.hpp"

namespace dg {
namespace {

constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) buffer, gfx9 family

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, kRsrcWord3);
}

// cache policy of the split-K partial stores and loads: coherent at agent
// scope (the XCDs' L2 caches are not kept coherent with each other)
constexpr int kCoherent = 16;  // sc1
// cache policy of the weight loads when one row tile covers M, so every
// weight line is read by exactly one workgroup: non-temporal (nt)
constexpr int kStream = 2;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int BM, int WN, int P, bool ACC, bool UE, bool NT>
__global__ void __launch_bounds__(256) fp8_gemm_skinny_kernel(GemmParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NW = 4;
  constexpr int TM = BM / 16;
  constexpr int TN = WN / 16;
  constexpr int BN = NW * WN;
  constexpr int A_INS = BM / 8 / NW;  // 1 KB buffer-to-LDS loads per wave per K block: A
  constexpr int B_INS = 2 * TN;       // ... and this wave's own B columns
  constexpr int L_STEP = A_INS + 1 + B_INS;
  constexpr int TG = 4;  // 16-row tiles whose fragments, MFMAs and promotions are batched
  static_assert(BM == 64 || BM == 128, "BM");
  static_assert(WN == 16 || WN == 32, "WN");
  static_assert(P == 4 || P == 6 || P == 8, "ring depth");
  static_assert((P - 1) * L_STEP < 64, "vmcnt range");
  static_assert(!(ACC && UE), "the accumulating form has fp32 scales");

  // ring slots are separate arrays so the compiler can tell DMA targets from
  // the slots being read; slots 4..7 exist only for deeper rings
  constexpr int SA = BM * 128;  // A slot bytes
  constexpr int SB = BN * 128;  // B slot bytes: WN columns per wave
  constexpr int SS = NW * 64;   // alpha: 64 rows per wave, only the tile's BM rows are read
#define SK_DECL(i, deep)                                                                                   \
  __shared__ __attribute__((aligned(1024))) uint8_t sA##i[(deep) ? SA : 16];                               \
  __shared__ __attribute__((aligned(1024))) uint8_t sB##i[(deep) ? SB : 16];                               \
  __shared__ __attribute__((aligned(256))) float sS##i[(deep) ? SS : 4];
  SK_DECL(0, true)
  SK_DECL(1, true)
  SK_DECL(2, true)
  SK_DECL(3, true)
  SK_DECL(4, P > 4)
  SK_DECL(5, P > 4)
  SK_DECL(6, P > 6)
  SK_DECL(7, P > 6)
#undef SK_DECL
  __shared__ int last_split;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4;

  // workgroup id -> (row tile, column tile, split): the row tiles of one
  // (column tile, split) unit are 8 ids apart (same XCD under round-robin
  // dispatch); units beyond the last one (padding of the grid to a multiple
  // of 8 units) exit at once
  const int S = p.splits;
  const int bid = (int)blockIdx.x;
  const int r8 = bid >> 3;
  const int mt = r8 % p.m_tiles;
  const int unit = (r8 / p.m_tiles) * 8 + (bid & 7);
  if (unit >= p.n_tiles * S) return;
  const int split = unit % S;  // the splits of a tile run side by side
  const int nt = unit / S;
  const int m0 = mt * BM;
  const int K = p.K;
  const int N = p.N;
  const int M = (int)p.rows;
  const int KB = K >> 7;
  const int KW = (KB + 3) >> 2;  // UE8M0: packed words (four K blocks) per scale row
  const int NB = (N + 127) >> 7;
  const int kb_lo = split * p.kb_per_split;
  const int kb_hi = kb_lo + p.kb_per_split < KB ? kb_lo + p.kb_per_split : KB;
  const int nsteps = kb_hi - kb_lo;  // >= 1 by construction of the split
  // Each tile walks its K blocks starting at a tile-dependent offset, so the
  // workgroups of an XCD do not all read the same A lines at the same moment
  // (every workgroup reads all of A).  The order is a fixed function of the
  // tile, so results are deterministic.
  const int rot = (int)(((unsigned)(nt * 5 + mt * 3)) % (unsigned)nsteps);
  const int n0 = nt * BN;
  const int wn0 = n0 + wave * WN;

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A + (int64_t)m0 * K, (uint32_t)(M - m0 < BM ? M - m0 : BM) * (uint32_t)K);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B, (uint32_t)N * (uint32_t)K);
  // alpha rows are sfa_ld apart (the row stride of the caller's [K/128][rows]
  // array); the range ends after this launch's last row of the last K block
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(p.sfa + m0, ((uint32_t)p.sfa_ld * (uint32_t)((UE ? KW : KB) - 1) + (uint32_t)(M - m0)) * 4u);
  // zero-length ranges: loads for the padding steps past the split's last
  // block read zeros and touch no memory
  const __amdgpu_buffer_rsrc_t ra0 = make_rsrc(p.A, 0);
  const __amdgpu_buffer_rsrc_t rb0 = make_rsrc(p.B, 0);
  const __amdgpu_buffer_rsrc_t rs0 = make_rsrc(p.sfa, 0);

  // Every 1 KB buffer-to-LDS load fills 8 LDS rows of 128 bytes: lane l
  // writes row l / 8, position l % 8, and loads K chunk (l % 8) ^ (l / 8) of
  // its source row, so 16-byte chunk c of LDS row r holds K chunk c ^ (r % 8).
  const int dma_chunk = ((lane & 7) ^ ((lane >> 3) & 7)) << 4;
  // A: instruction i of this wave fills slot rows 8 (4 i + wave) + lane / 8;
  // rows at or past M fall outside A's buffer range and read as zeros
  const uint32_t a_src = (uint32_t)(8 * wave + (lane >> 3)) * (uint32_t)K + (uint32_t)dma_chunk;
  const uint32_t a_stride = 8u * NW * (uint32_t)K;
  // alpha: wave w loads rows 64 w + lane of the block; rows past the tile are
  // never read (one load per wave keeps the counts equal)
  const uint32_t s_src = (uint32_t)(wave * 64 + lane) * 4u;
  // B is the MFMA's row operand: row i of column tile j is weight row
  // wn0 + (i / 4) * 4 TN + 4 j + i % 4, so that lane l's outputs (rows
  // 4 (l / 16) + v of every tile j) are the 4 TN consecutive columns
  // wn0 + (l / 16) * 4 TN + [0, 4 TN) of one output row.  Tile j of this wave
  // occupies 16 LDS rows (two loads, h = 0, 1: rows 8 h + lane / 8) of the slot.
  uint32_t b_src[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = 8 * h + (lane >> 3);
    b_src[h] = (uint32_t)(wn0 + (i >> 2) * 4 * TN + (i & 3)) * (uint32_t)K + (uint32_t)dma_chunk;
  }
  const uint32_t b_tile = 4u * (uint32_t)K;

  // fragment reads: row 16 t + lane % 16 of a slot, chunks q and q + 4
  const uint32_t fr_lo = (uint32_t)((lane & 15) * 128 + ((q ^ (lane & 7)) << 4));
  const uint32_t fr_hi = (uint32_t)((lane & 15) * 128 + (((q + 4) ^ (lane & 7)) << 4));

  // weight scale row of this wave's columns (WN <= 32 columns lie in one
  // 128-column block, whatever the order of rows inside the wave), read
  // through the scalar cache
  int nblk = wn0 >> 7;
  nblk = nblk < NB ? nblk : NB - 1;
  const DG_CONST float* sfb_w;
  {
    const uint64_t a = reinterpret_cast<uint64_t>(p.sfb + nblk * (UE ? KW : KB));
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    sfb_w = (const DG_CONST float*)(((uint64_t)hi << 32) | lo);
  }

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#define SK_SLOT(arr, st)                                                                                   \
  ((st) == 0 ? arr##0 : (st) == 1 ? arr##1 : (st) == 2 ? arr##2 : (st) == 3 ? arr##3 : (st) == 4 ? arr##4  \
   : (st) == 5 ? arr##5 : (st) == 6 ? arr##6 : arr##7)

  // K block of step jj (jj < nsteps) in the rotated order
#define SK_KB(jj_) (kb_lo + ((jj_) + rot < nsteps ? (jj_) + rot : (jj_) + rot - nsteps))
  // A, alpha and this wave's B of step jj_'s K block into ring slot st_
  // (zeros for padding steps, jj_ >= nsteps)
#define SK_ISSUE(st_, jj_)                                                                                 \
  do {                                                                                                     \
    const bool in_ = (jj_) < nsteps;                                                                       \
    const int kb_ = in_ ? SK_KB(jj_) : 0;                                                                  \
    const __amdgpu_buffer_rsrc_t ra_ = in_ ? ra : ra0;                                                     \
    const __amdgpu_buffer_rsrc_t rb_ = in_ ? rb : rb0;                                                     \
    const __amdgpu_buffer_rsrc_t rs_ = in_ ? rs : rs0;                                                     \
    _Pragma("unroll") for (int i_ = 0; i_ < A_INS; ++i_)                                                   \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra_, (DG_LDS void*)(SK_SLOT(sA, st_) + (i_ * NW + wave) * 1024), \
                                                 16, a_src + i_ * a_stride, (kb_) << 7, 0, 0);             \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_, (DG_LDS void*)(SK_SLOT(sS, st_) + wave * 64), 4, s_src,  \
                                             (UE ? (kb_) >> 2 : (kb_)) * p.sfa_ld * 4, 0, 0);              \
    _Pragma("unroll") for (int j_ = 0; j_ < TN; ++j_)                                                      \
      _Pragma("unroll") for (int h_ = 0; h_ < 2; ++h_)                                                     \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                          \
            rb_, (DG_LDS void*)(SK_SLOT(sB, st_) + (wave * TN + j_) * 2048 + h_ * 1024), 16,               \
            b_src[h_] + j_ * b_tile, (kb_) << 7, 0, NT ? kStream : 0);                                     \
  } while (0)

  // Step j (the j-th K block in rotated order, ring slot st_ = j % P):
  //   1. wait until this wave's loads of block j have landed (the P - 2 later
  //      blocks may remain in flight) and its LDS reads of step j - 1 have
  //      returned; one s_barrier makes block j visible to all waves and frees
  //      the slot of block j - 1;
  //   2. refill that slot with block j + P - 1;
  //   3. read this wave's B fragments; per group of four 16-row tiles read
  //      the A fragments and alpha, one MFMA per (row tile, column tile), then
  //      the promotions with alpha * beta (rows at or past M hold zeros and
  //      are never stored).
  // The step count is padded to a multiple of P; padding steps load zeros,
  // so they add exactly 0 (alpha = 0 there), and every step issues the same
  // loads, which keeps the wait counts the same.
#define SK_FRAG(base_)                                                                                     \
  ([&]() {                                                                                                 \
    const uint4 lo_ = *reinterpret_cast<const uint4*>((base_) + fr_lo);                                    \
    const uint4 hi_ = *reinterpret_cast<const uint4*>((base_) + fr_hi);                                    \
    return i32x8{(int)lo_.x, (int)lo_.y, (int)lo_.z, (int)lo_.w, (int)hi_.x, (int)hi_.y, (int)hi_.z, (int)hi_.w}; \
  }())
#define SK_STEP(st_, j_)                                                                                   \
  do {                                                                                                     \
    const int kbj_ = (j_) < nsteps ? SK_KB(j_) : kb_lo;                                                    \
    /* fp32 scales: beta of the block; UE8M0: the block's codes are byte kbj_ % 4 of the packed words */   \
    const float beta_ = UE ? 1.f : sfb_w[kbj_];                                                            \
    const int ash_ = 8 * (kbj_ & 3);                                                                       \
    const int bcode_ = UE ? __builtin_bit_cast(int, sfb_w[kbj_ >> 2]) >> ash_ : 0;                        \
    (void)ash_;                                                                                            \
    (void)bcode_;                                                                                          \
    wait_vmcnt<(P - 2) * L_STEP>();                                                                        \
    wait_lgkmcnt0();                                                                                       \
    __builtin_amdgcn_s_barrier();                                                                          \
    SK_ISSUE(((st_) + P - 1) % P, (j_) + P - 1);                                                          \
    const uint8_t* as_ = SK_SLOT(sA, st_);                                                                 \
    const uint8_t* bs_ = SK_SLOT(sB, st_) + wave * TN * 2048;                                              \
    const float* ss_ = SK_SLOT(sS, st_);                                                                   \
    i32x8 bf_[TN];                                                                                         \
    _Pragma("unroll") for (int j2_ = 0; j2_ < TN; ++j2_) bf_[j2_] = SK_FRAG(bs_ + j2_ * 2048);             \
    _Pragma("unroll") for (int g_ = 0; g_ < TM; g_ += TG) {                                                \
      i32x8 af_[TG];                                                                                       \
      float sc_[TG]; /* fp32 scales: alpha * beta of the row tile's rows */                                \
      int acode_[TG]; /* UE8M0: the rows' alpha codes in byte 0 */                                         \
      f32x4 t_[TG][TN];                                                                                    \
      _Pragma("unroll") for (int i_ = 0; i_ < TG; ++i_) {                                                  \
        af_[i_] = SK_FRAG(as_ + (g_ + i_) * 2048);                                                         \
        const float al_ = ss_[(g_ + i_) * 16 + (lane & 15)];                                               \
        if constexpr (UE) acode_[i_] = __builtin_bit_cast(int, al_) >> ash_;                               \
        else sc_[i_] = al_ * beta_;                                                                        \
      }                                                                                                    \
      _Pragma("unroll") for (int i_ = 0; i_ < TG; ++i_)                                                    \
        _Pragma("unroll") for (int j2_ = 0; j2_ < TN; ++j2_) {                                             \
          if constexpr (UE) /* alpha and beta applied, and the scaled block product added to the */        \
            /* accumulator, by the matrix cores (exact powers of two): the promotion in one instruction */  \
            acc[g_ + i_][j2_] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(                          \
                bf_[j2_], af_[i_], acc[g_ + i_][j2_], 0, 0, 0, bcode_, 0, acode_[i_]);                      \
          else                                                                                             \
            t_[i_][j2_] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(                                \
                bf_[j2_], af_[i_], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);                           \
        }                                                                                                  \
      if constexpr (!UE)                                                                                   \
        _Pragma("unroll") for (int i_ = 0; i_ < TG; ++i_)                                                  \
          _Pragma("unroll") for (int j2_ = 0; j2_ < TN; ++j2_)                                             \
            _Pragma("unroll") for (int v_ = 0; v_ < 4; ++v_)                                               \
              acc[g_ + i_][j2_][v_] = __builtin_fmaf(t_[i_][j2_][v_], sc_[i_], acc[g_ + i_][j2_][v_]);     \
    }                                                                                                      \
  } while (0)

  // prologue: steps 0 .. P-2 into slots 0 .. P-2
  _Pragma("unroll") for (int t = 0; t + 1 < P; ++t) SK_ISSUE(t, t);

  // one fully unrolled ring cycle per iteration, no tail: a tail after the
  // loop would hide from the compiler which ring slot each pending load
  // targets and cost conservative waits
  for (int j = 0; j < nsteps; j += P) {
    _Pragma("unroll") for (int t = 0; t < P; ++t) SK_STEP(t, j + t);
  }
  wait_vmcnt<0>();  // no LDS loads may be in flight past this point

#undef SK_STEP
#undef SK_FRAG
#undef SK_ISSUE
#undef SK_KB
#undef SK_SLOT

  if (S > 1) {
    // Split K.  Partial of this split in fragment order: for split s, tile
    // (mt, nt) and wave w, fragment (i, j) of lane l sits at float offset
    // ((((s * m_tiles + mt) * n_tiles + nt) * 4 + w) * TM * TN + i * TN + j) * 256 + 4 l.
    // Ordering (the same argument as the persistent kernel's tail pieces):
    // the partial stores and loads carry sc1, which is how the compiler lowers
    // relaxed agent-scope atomic stores and loads on gfx950, so each access
    // is coherent across the XCDs' L2 caches.  Each wave waits (vmcnt(0))
    // until its sc1 stores are acknowledged at that coherence point before
    // the barrier that precedes the relaxed counter increment; the last split
    // issues its sc1 loads only after its increment has returned.  The
    // write-back / invalidate of the L2 that an agent-scope release / acquire
    // adds concern data cached non-coherently, which these accesses never are.
    const int tiles = p.m_tiles * p.n_tiles;
    const int tile = mt * p.n_tiles + nt;
    const uint32_t frag_bytes = (uint32_t)TM * TN * 1024u;  // one wave's fragments
    const uint32_t split_bytes = (uint32_t)tiles * NW * frag_bytes;
    // counters at the workspace start, partials after them
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(reinterpret_cast<uint8_t*>(p.ws) + kWsCounterBytes, (uint32_t)S * split_bytes);
    const uint32_t w_off = ((uint32_t)tile * NW + wave) * frag_bytes + (uint32_t)lane * 16u;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int jj = 0; jj < TN; ++jj)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][jj]), rw,
                                               w_off + (uint32_t)(i * TN + jj) * 1024u, (uint32_t)split * split_bytes,
                                               kCoherent);
    wait_vmcnt<0>();
    __syncthreads();
    unsigned int* counters = reinterpret_cast<unsigned int*>(p.ws);
    if (tid == 0)
      last_split = __hip_atomic_fetch_add(&counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   (unsigned int)(S - 1);
    __syncthreads();
    if (!last_split) return;
#define SK_LDP(s_, i_, j_)                                                                                 \
  __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(                                         \
                                rw, w_off + (uint32_t)((i_) * TN + (j_)) * 1024u, (uint32_t)(s_) * split_bytes, kCoherent))
    // sum of the splits' fragments in split order, into acc: the loads of up
    // to SB splits are in flight at once (one round trip per batch), the
    // additions keep the order 0, 1, 2, ...
    constexpr int SB = TM * TN <= 4 ? 8 : (TM * TN <= 8 ? 4 : 2);
    for (int k0 = 0; k0 < S; k0 += SB) {
      f32x4 t[SB][TM][TN];
#pragma unroll
      for (int b = 0; b < SB; ++b)
        if (k0 + b < S) {
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int jj = 0; jj < TN; ++jj) t[b][i][jj] = SK_LDP(k0 + b, i, jj);
        }
#pragma unroll
      for (int b = 0; b < SB; ++b)
        if (k0 + b < S) {
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int jj = 0; jj < TN; ++jj) acc[i][jj] = (k0 + b == 0) ? t[b][i][jj] : acc[i][jj] + t[b][i][jj];
        }
    }
#undef SK_LDP
    if (tid == 0)  // ready for the next call on this workspace
      __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // epilogue: for row tile i, lane l holds output row m0 + 16 i + l % 16 and
  // its columns wn0 + q * 4 TN + 4 j + v, i.e. 4 TN consecutive bf16 (8 or 16
  // bytes per store).  N is a multiple of 16 and 4 TN divides 16, so a lane's
  // columns are all inside N or all outside.
  const int c0 = wn0 + q * 4 * TN;
  if constexpr (ACC) {
    // accumulating form: fp32 D = C + acc (4 TN consecutive floats per row
    // tile); every C load before the first store, since C may be D itself
    f32x4 cv[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = m0 + i * 16 + (lane & 15);
#pragma unroll
      for (int jj = 0; jj < TN; ++jj)
        cv[i][jj] = (r < M && c0 < N && p.Cacc)
                        ? *reinterpret_cast<const f32x4*>(p.Cacc + (int64_t)r * N + c0 + 4 * jj)
                        : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = m0 + i * 16 + (lane & 15);
      if (r >= M || c0 >= N) continue;
#pragma unroll
      for (int jj = 0; jj < TN; ++jj)
        *reinterpret_cast<f32x4*>(p.Dacc + (int64_t)r * N + c0 + 4 * jj) = acc[i][jj] + cv[i][jj];
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int r = m0 + i * 16 + (lane & 15);
    if (r >= M || c0 >= N) continue;
    uint16_t* dst = p.D + (int64_t)r * N + c0;
    if (TN == 1) {
      uint2 o;
      o.x = pack_bf16x2(acc[i][0][0], acc[i][0][1]);
      o.y = pack_bf16x2(acc[i][0][2], acc[i][0][3]);
      *reinterpret_cast<uint2*>(dst) = o;
    } else {
      uint4 o;
      uint32_t w[4];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        w[2 * jj] = pack_bf16x2(acc[i][jj][0], acc[i][jj][1]);
        w[2 * jj + 1] = pack_bf16x2(acc[i][jj][2], acc[i][jj][3]);
      }
      o.x = w[0];
      o.y = w[1];
      o.z = w[2];
      o.w = w[3];
      *reinterpret_cast<uint4*>(dst) = o;
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

template <int BM, int WN, int P, bool NT>
void launch_skinny_form(bool ue, const GemmParams& p, int64_t grid, hipStream_t stream) {
  if (ue)
    hipLaunchKernelGGL((fp8_gemm_skinny_kernel<BM, WN, P, false, true, NT>), dim3((unsigned)grid), dim3(256), 0, stream, p);
  else if (p.Dacc)
    hipLaunchKernelGGL((fp8_gemm_skinny_kernel<BM, WN, P, true, false, NT>), dim3((unsigned)grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((fp8_gemm_skinny_kernel<BM, WN, P, false, false, NT>), dim3((unsigned)grid), dim3(256), 0, stream, p);
}

template <int BM, int WN, int P>
hipError_t launch_skinny_cfg(bool ue, const GemmParams& p, hipStream_t stream) {
  const int64_t units = (int64_t)p.n_tiles * p.splits;
  const int64_t grid = (units + 7) / 8 * 8 * p.m_tiles;
  if (grid <= 0) return hipSuccess;
  // M <= 64 (one 64-row tile): the weights stream past once with the
  // non-temporal policy.  Where two row tiles share the weights, or one
  // 128-row tile reads them, the default policy measured faster.
  if constexpr (BM == 64) {
    if (p.m_tiles == 1) {
      launch_skinny_form<BM, WN, P, true>(ue, p, grid, stream);
      return hipGetLastError();
    }
  }
  launch_skinny_form<BM, WN, P, false>(ue, p, grid, stream);
  return hipGetLastError();
}

}  // namespace

size_t skinny_workspace_bytes(int bm, int m_tiles, int n_tiles, int wn, int splits) {
  if (splits <= 1) return 0;
  // the counter area, then fp32 partials of bm x 4wn tiles
  return kWsCounterBytes + (size_t)splits * m_tiles * n_tiles * bm * 4 * wn * 4;
}

hipError_t launch_gemm_skinny(int bm, int wn, int depth, bool ue, const GemmParams& p, hipStream_t stream) {
  if (bm == 64 && wn == 16)
    return depth == 8 ? launch_skinny_cfg<64, 16, 8>(ue, p, stream) : launch_skinny_cfg<64, 16, 4>(ue, p, stream);
  if (bm == 64)
    return depth == 6 ? launch_skinny_cfg<64, 32, 6>(ue, p, stream) : launch_skinny_cfg<64, 32, 4>(ue, p, stream);
  return wn == 16 ? launch_skinny_cfg<128, 16, 6>(ue, p, stream) : launch_skinny_cfg<128, 32, 4>(ue, p, stream);
}

}  // namespace dg
