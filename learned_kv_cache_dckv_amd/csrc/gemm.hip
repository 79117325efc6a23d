// Transform stages of the DCKV codec on gfx950: bf16 MFMA GEMMs with fp32
// accumulation and fused epilogues.
//
// Source: DCKV digest page ("DCKV: Learned Transform Coding of the Prompt KV
// Cache in Hybrid Language Models"), "How it works":
//   - Transform: one shared basis maps every 6,144-dim row to 2,048
//     coefficients; a small nonlinear correction (one hidden layer of 256
//     GELU units) is added on the synthesis side;
//   - Conditional entropy models: even positions take their code means from
//     the prompt token's input embedding, odd positions also from the decoded
//     coefficients of both neighbours (a 1-D checkerboard, two passes);
//   - first paragraph: the codec sees the keys without their rotary position
//     embedding, and the decoder rotates them again at the end.
//
// Every GEMM here is C[m][n] = sum_k A[m][k] * B[n][k] with both operands
// k-contiguous (token rows times weight rows).  One workgroup of four wave64s
// owns a 256x256 tile; each wave a 128x128 sub-tile held as 4x4 blocks of
// v_mfma_f32_32x32x16_bf16 accumulators (256 fp32 per lane); the 32x32 form
// keeps the matrix cores busy with a single wave per SIMD.  Operand tiles of
// 256 rows x 64 k (whole 128-byte lines) are copied global -> LDS by the
// direct 16-byte LDS loads of gfx950 (no register staging) into two stages;
// one barrier per k-tile.  Chunk c of row r is stored at c ^ ((r >> 1) & 7),
// so the 16 lanes served together by one LDS pass read 16 distinct 16-byte
// bank groups.  Fragments of the next k-step are read from LDS while the
// current k-step's MFMAs run.  Workgroups are mapped to tiles so that the
// tiles one XCD runs at once share their operand panels in that XCD's L2.
//
// Lane l of a 32x32 accumulator block holds column l%32 and, in register
// group g (registers 4g..4g+3), rows 8g + 4*(l/32) .. +3: a quad of 4
// consecutive rows.  The checkerboard neighbours of a row are in the same
// quad (rows 4k+1: 4k and 4k+2) or, for row 4k+3, in the first row of the
// next quad, held by lane l^32 (same group, or the next group / next block).
//
// The embedding mean H E[tok] depends on the token id alone, so the plan
// holds it for the whole vocabulary (computed once by k_mean_table, fp32).
// The kernels:
//   mean table  H E[v] for every token id v -> fp32 [vocab][C], columns in the
//               plan's rank order (active components, then dropped ones)
//   quantise    analysis GEMM; epilogue: even rows r = (y - mu)/step,
//               q = rint(r), yhat = mu + q step; then odd rows with
//               mu += a (yhat_{j-1} + yhat_{j+1}); mu comes from the table
//               straight into registers, six accumulator blocks ahead; the
//               first row of the lower wave crosses waves through LDS, the
//               last odd row of a tile is finished by a small fix-up kernel
//   dequant     no GEMM: yhat = mu + q step in the same two passes, streamed
//               row by row from the table, the codes and the escape records
//               -> bf16 yhat_b
//   w1          exact-erf GELU -> bf16 h_b
//   synthesis   rotate-half RoPE on key heads; the tile's columns are ordered
//               so that every pair (d, d+128) sits in one lane and register
//               of blocks nb and nb+2 -> bf16 rows
// Synthesis is persistent: a wave keeps most of its bf16 output tile in
// registers and stores it during the next tile's main loop.
#include <cmath>

#include <vector>

#include "dckv_internal.h"

namespace dckv {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef const void __attribute__((address_space(1))) *gptr_t;
typedef void __attribute__((address_space(3))) *lptr_t;

constexpr int kThreads = 256;
constexpr int kStages = 2;
constexpr int kRowBytes = kBK * 2;                        // 128 B per staged row
constexpr int kStageBytes = (kBM + kBN) * kRowBytes;      // 64 KiB per stage
// after the main loop the quantiser reuses LDS for its token ids (512 B per
// wave) and its even rows' yhat (32 KiB per wave); the row-0 exchange between
// the two wave rows sits above both
constexpr int kQuantEpiBytes = 4 * 512 + 4 * 16 * 2 * 64 * 16;
constexpr int kXchOff = kQuantEpiBytes > kStages * kStageBytes ? kQuantEpiBytes : kStages * kStageBytes;
constexpr int kLdsBytes = kXchOff + 2 * 256 * 4;
static_assert(kStages * kStageBytes <= kXchOff, "stages must not overlap the exchange area");
static_assert(kLdsBytes <= 160 * 1024, "LDS budget of one workgroup");
constexpr float kQLimit = 2147483520.0f;  // largest float below 2^31

__device__ __forceinline__ void set_status(int32_t *st, int code) { atomicCAS(st, 0, code); }

// One read of the status word per workgroup, so that every wave of the
// workgroup takes the same early exit (other workgroups may set it meanwhile).
__device__ __forceinline__ bool wg_stop(const int32_t *st) {
  __shared__ int s_stop;
  if (threadIdx.x == 0) s_stop = *reinterpret_cast<const volatile int32_t *>(st);
  __syncthreads();
  return s_stop != 0;
}

// A load through a global (address space 1) pointer.
template <class T>
__device__ __forceinline__ T gload(const T *p) {
  return *(const T __attribute__((address_space(1))) *)p;
}

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even: the conversion instruction of gfx950
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;

// two fp32 -> two bf16 in one word (a in the low half), one instruction
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// XCD-aware tile order: workgroup b runs on XCD b % 8; each XCD gets a
// contiguous run of tile indices.  Tile index t walks column groups of up to 8
// tiles, row bands inside a group, columns inside a band, so the 32 tiles an
// XCD runs at once form a 4 x 8 block: per k-tile they read 4 row panels and 8
// column panels, shared through that XCD's L2.
__device__ __forceinline__ void tile_of(int b, int total, int n_nt, int &mt, int &nt) {
  const int q = total >> 3, r = total & 7, x = b & 7, k = b >> 3;
  const int t = x < r ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
  const int gw = n_nt < 8 ? n_nt : 8;     // column tiles per group (n_nt is 1..8 or a multiple of 8)
  const int n_mt = total / n_nt;
  const int grp = t / (gw * n_mt), rem = t - grp * gw * n_mt;
  mt = rem / gw;
  nt = grp * gw + (rem - mt * gw);
}

// ---------------------------------------------------------------------------
// operand staging and the MFMA main loop
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;

struct Operand {
  const char *p0, *p1;  // two k-ranges (k-tiles [0, split) and the rest)
  uint32_t rb0, rb1;    // row bytes of each source
  int split;
  uint32_t row[8];      // source rows staged by this lane: tile rows wave*64 + 8i + lane/8
};

__device__ __forceinline__ void set_sources(Operand &op, const void *p0, uint32_t rb0, const void *p1, uint32_t rb1,
                                            int split) {
  op.p0 = reinterpret_cast<const char *>(p0);
  op.p1 = reinterpret_cast<const char *>(p1);
  op.rb0 = rb0;
  op.rb1 = rb1;
  op.split = split;
}

// Where the loads of one k-tile of one operand come from: a buffer resource
// over its source (no stride, full 32-bit range), the k offset (a scalar) and
// the source's row bytes.  k-tiles at or past KT get a resource with no range,
// so their loads move no data.
struct TileSrc {
  rsrc_t r;
  uint32_t soff, rb;
};

// kKV: the k-tiles alternate in runs of 8 (one layer's two key heads, then
// its two value heads); key runs come from p0, a [rows][6 * 512] key copy,
// value runs from p1 at their own columns (split unused).
template <bool kKV = false>
__device__ __forceinline__ TileSrc tile_src(const Operand &op, int kt, int KT) {
  const bool s0 = kKV ? ((kt >> 3) & 1) == 0 : kt < op.split;
  // base and range are wave-uniform: keep them in scalar registers
  const uint64_t b = reinterpret_cast<uint64_t>(s0 ? op.p0 : op.p1);
  // (readfirstlane returns int: zero-extend each half, never sign-extend)
  const uint64_t bu = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b) |
                      ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32);
  const int nrec = __builtin_amdgcn_readfirstlane(kt < KT ? -1 : 0);
  TileSrc t;
  t.r = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(bu), (short)0, nrec, 0x00020000);
  t.rb = s0 ? op.rb0 : op.rb1;
  if (kKV)
    t.soff = (uint32_t)(s0 ? (kt >> 4) * 8 + (kt & 7) : kt) * kRowBytes;
  else
    t.soff = (uint32_t)(s0 ? kt : kt - op.split) * kRowBytes;
  return t;
}

// Direct load i (0..7) of one operand's k-tile (256 rows x 64 k) into its LDS
// region: each wave stages 64 rows, one load writing 1 KiB = 8 rows of 128
// bytes, so every load covers whole 128-byte lines.  Lane l fills physical
// chunk l & 7 of row l / 8, which holds logical chunk (l & 7) ^ ((row >> 1) & 7);
// for the rows of load i that is (l & 7) ^ (4 (i & 1) + l / 16).
__device__ __forceinline__ void load_rows(const Operand &op, const TileSrc &t, int i, char *region, int wave, int lane) {
  const uint32_t c = (uint32_t)(((lane & 7) ^ (((i & 1) << 2) + (lane >> 4))) << 4);
  const uint32_t voff = op.row[i] * t.rb + c;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(t.r, (lptr_t)(region + (wave * 64 + i * 8) * kRowBytes), 16, voff, t.soff, 0,
                                           0);
}

__device__ __forceinline__ bf16x8 frag(const char *region, int row, int c) {
  return *reinterpret_cast<const bf16x8 *>(region + row * kRowBytes + ((c ^ ((row >> 1) & 7)) << 4));
}

struct Frags {
  bf16x8 a[4], b[4];
};

// Fragments of k-step ks (16 k) of a stage: chunk 2 ks + lane / 32.
__device__ __forceinline__ void read_frags(Frags &f, const char *stage, int ks, int lane, int wm, int wn) {
  const int c = ks * 2 + (lane >> 5);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) f.a[mb] = frag(stage, wm * 128 + mb * 32 + (lane & 31), c);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) f.b[nb] = frag(stage + kBM * kRowBytes, wn * 128 + nb * 32 + (lane & 31), c);
}

// One k-step in a fixed instruction order: the 16 MFMAs of fragments f; after
// each of the first 8, one LDS read of the fragments g of k-step gks of gstage;
// after every second MFMA, direct load (i / 2) of `load` (a no-op where a
// k-step issues none).  Spreading the loads keeps the vector memory queue from
// backing up into the MFMA issue.
template <class L>
__device__ __forceinline__ void kstep(f32x16 (&acc)[4][4], const Frags &f, Frags &g, const char *gstage, int gks,
                                      int lane, int wm, int wn, L &&load) {
  const int c = gks * 2 + (lane >> 5);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int mb = i >> 2, nb = i & 3;
    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[mb], f.b[nb], acc[mb][nb], 0, 0, 0);
    if (i < 4) g.a[i] = frag(gstage, wm * 128 + i * 32 + (lane & 31), c);
    else if (i < 8) g.b[i - 4] = frag(gstage + kBM * kRowBytes, wn * 128 + (i - 4) * 32 + (lane & 31), c);
    if (i & 1) load(i >> 1);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Wait until at most n of this wave's direct loads are in flight and all of
// its LDS reads are done, then meet the other waves.  s_waitcnt fields:
// vmcnt[3:0] and [15:14], expcnt[6:4] (7 = no wait), lgkmcnt[11:8] (0 = wait).
template <int n>
__device__ __forceinline__ void tile_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((n & 15) | 0x70 | ((n >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Two LDS stages; k-tile t lives in stage t % 2 and is consumed in four
// k-steps.  Before the last one, every wave waits for its loads of k-tile
// kt + 1 and the workgroup meets: k-tile kt + 1 is then visible and stage
// kt % 2 has been read in full.  The last k-step reads the first fragments of
// k-tile kt + 1 and issues the A loads of k-tile kt + 2 into the free stage; the
// first k-step of the next tile issues its B loads.
struct NoSide {
  __device__ void operator()(int) const {}
};

// kPeel > 0: the first kPeel k-tiles are unrolled and call side(8 kt + i),
// i = 0..7, spread over their third k-step (work with compile-time indices,
// such as stores of registers held from a previous tile); needs KT >= kPeel.
template <bool kPinAcc = true, int kPeel = 0, bool kKV = false, class S = NoSide>
__device__ __forceinline__ void mainloop(const Operand &A, const Operand &B, int KT, f32x16 (&acc)[4][4],
                                         char *lds, S &&side = S()) {
  // the wave index in a scalar register: LDS destinations of the direct loads
  // (M0) must be wave-uniform
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  {
    const TileSrc a0 = tile_src<kKV>(A, 0, KT), b0 = tile_src(B, 0, KT);
#pragma unroll
    for (int i = 0; i < 8; ++i) load_rows(A, a0, i, lds, wave, lane);
#pragma unroll
    for (int i = 0; i < 8; ++i) load_rows(B, b0, i, lds + kBM * kRowBytes, wave, lane);
  }
  TileSrc ta = tile_src<kKV>(A, 1, KT), tb = tile_src(B, 1, KT);
#pragma unroll
  for (int i = 0; i < 8; ++i) load_rows(A, ta, i, lds + kStageBytes, wave, lane);
  tile_barrier<8>();  // k-tile 0 has landed
  Frags f0, f1;
  read_frags(f0, lds, 0, lane, wm, wn);
  const auto none = [](int) {};
  auto body = [&](int kt, auto &&sidek) {
    char *cur = lds + (kt & 1) * kStageBytes;
    char *nxt = lds + ((kt + 1) & 1) * kStageBytes;
    kstep(acc, f0, f1, cur, 1, lane, wm, wn, [&](int i) { load_rows(B, tb, i, nxt + kBM * kRowBytes, wave, lane); });
    kstep(acc, f1, f0, cur, 2, lane, wm, wn, sidek);
    kstep(acc, f0, f1, cur, 3, lane, wm, wn, none);
    tile_barrier<0>();
    ta = tile_src<kKV>(A, kt + 2, KT);
    tb = tile_src(B, kt + 2, KT);
    kstep(acc, f1, f0, nxt, 0, lane, wm, wn, [&](int i) { load_rows(A, ta, i, cur, wave, lane); });
  };
#pragma unroll
  for (int kt = 0; kt < kPeel; ++kt) body(kt, [&](int i) { side(8 * kt + i); });
#pragma unroll 1
  for (int kt = kPeel; kt < KT; ++kt) body(kt, none);
  __syncthreads();
  // The accumulators leave the loop in AGPRs; epilogues copy them to VGPRs one
  // block at a time (an epilogue that needs them in VGPRs would otherwise have
  // all 256 copied at the loop exit, and the loop's own registers spilled).
  if (kPinAcc) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) asm volatile("" : "+a"(acc[i][j]));
  }
}

// The lane id, opaque to the optimiser: epilogue address arithmetic derived
// from it cannot be hoisted above the main loop, where it would hold
// registers for the loop's whole duration.
__device__ __forceinline__ int epilogue_lane() {
  int l = threadIdx.x & 63;
  asm volatile("" : "+v"(l));
  return l;
}

// One accumulator block in VGPRs, copied where it is used.
__device__ __forceinline__ f32x16 acc_block(const f32x16 (&acc)[4][4], int mb, int nb) {
  f32x16 b = acc[mb][nb];
  asm volatile("" : "+v"(b));
  return b;
}


// Register v of an accumulator block, read out of its AGPR in place (the
// block is not copied to VGPRs as a whole).
__device__ __forceinline__ float acc_get(const f32x16 &b, int v) {
  float x;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(x) : "a"(b[v]));
  return x;
}

// Row (within the wave tile) of register v of block row mb in this lane.
__device__ __forceinline__ int acc_row(int mb, int v, int lane) { return mb * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

// the constant part of acc_row(): row of register v of block mb without the lane term
__device__ __forceinline__ constexpr int acc_crow(int mb, int v) { return mb * 32 + 8 * (v >> 2) + (v & 3); }

// ---------------------------------------------------------------------------
// operand setup helpers
// ---------------------------------------------------------------------------
// tile row staged by this lane in load i (0..7), matching load_rows()
__device__ __forceinline__ int staged_row(int i) { return (threadIdx.x >> 6) * 64 + i * 8 + ((threadIdx.x & 63) >> 3); }

// ---------------------------------------------------------------------------
// plan time: embedding-mean table  mtab[v][i] = sum_k E[v][k] H[perm[i]][k]
// ---------------------------------------------------------------------------
struct MeanTabP {
  const uint16_t *E, *H;
  const int32_t *perm;
  float *mtab;  // [vocab][kC]
  int vocab, n_mt, n_nt;
};

__global__ __launch_bounds__(kThreads, 1) void k_mean_table(MeanTabP P) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  int mt, nt;
  tile_of(blockIdx.x, P.n_mt * P.n_nt, P.n_nt, mt, nt);
  const int m0 = mt * kBM;
  const int n0 = nt * kBN;
  Operand A, B;
  set_sources(A, P.E, kEmb * 2, P.E, kEmb * 2, kEmb / kBK);
  set_sources(B, P.H, kEmb * 2, P.H, kEmb * 2, kEmb / kBK);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    A.row[i] = (uint32_t)min(m0 + staged_row(i), P.vocab - 1);
    B.row[i] = (uint32_t)P.perm[n0 + staged_row(i)];
  }
  f32x16 acc[4][4];
  mainloop(A, B, kEmb / kBK, acc, lds);
  const int lane = epilogue_lane(), wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const f32x16 b = acc_block(acc, mb, nb);
      const int col = n0 + wn * 128 + nb * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * 128 + acc_row(mb, v, lane);
        if (row < P.vocab) P.mtab[(size_t)row * kC + col] = b[v];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
}

// ---------------------------------------------------------------------------
// fit: C[m][n] = sum_k A[m][k] B[n][k] with fp32 output (bf16 operands, two
// k-ranges per operand, optional row gather for A)
// ---------------------------------------------------------------------------
// Two independent products may share one launch (workgroups [0, blocks0) do
// the first), so that small ones fill the chip together.
struct GemmF32Pair {
  GemmF32Args g0, g1;
  int blocks0;
};

__global__ __launch_bounds__(kThreads, 1) void k_gemm_f32(GemmF32Pair PP) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const bool second = (int)blockIdx.x >= PP.blocks0;
  const GemmF32Args &P = second ? PP.g1 : PP.g0;
  const int bid = second ? (int)blockIdx.x - PP.blocks0 : (int)blockIdx.x;
  int mt, nt;
  // k-slice ks of ksplit (single-source operands): k-tiles [ks KT, (ks + 1) KT)
  // into the output slice c + ks M ldc
  const int tiles = P.n_mt * P.n_nt;
  const int ks = bid / tiles;
  tile_of(bid - ks * tiles, tiles, P.n_nt, mt, nt);
  const int KT = P.KT / P.ksplit;
  const size_t koff = (size_t)ks * KT * kRowBytes;
  const int split = P.ksplit > 1 ? KT : P.split;
  const int m0 = mt * kBM, n0 = nt * kBN;
  Operand A, B;
  set_sources(A, reinterpret_cast<const char *>(P.a0) + koff, P.lda0, reinterpret_cast<const char *>(P.a1) + koff,
              P.lda1, split);
  set_sources(B, reinterpret_cast<const char *>(P.b0) + koff, P.ldb0, reinterpret_cast<const char *>(P.b1) + koff,
              P.ldb1, split);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = min(m0 + staged_row(i), P.M - 1);
    A.row[i] = (uint32_t)(P.arow ? P.arow[m] : m);
    B.row[i] = (uint32_t)min(n0 + staged_row(i), P.N - 1);
  }
  f32x16 acc[4][4];
  mainloop(A, B, KT, acc, lds);
  const int lane = epilogue_lane(), wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  float *const cs = P.c + (size_t)ks * P.M * P.ldc;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int col = n0 + wn * 128 + nb * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * 128 + acc_row(mb, v, lane);
        if (row < P.M && col < P.N) cs[(size_t)row * P.ldc + col] = acc_get(acc[mb][nb], v);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
}

// ---------------------------------------------------------------------------
// encode: analysis GEMM + quantiser (two checkerboard passes)
// ---------------------------------------------------------------------------
struct QuantP {
  const uint16_t *rows, *A;
  const uint16_t *keys;  // set: key heads from this pre-RoPE key copy [T][6 * 512], value heads from rows
  const int32_t *act, *tok;
  const float *step, *nbr;
  const float *qcol;  // [C_a padded][4]: step, 1 / step (0 past C_a), a, 0 of each rank
  const float *mtab;  // [vocab][kC] embedding means, columns in rank order
  uint32_t *sym32;
  uint32_t *esc_raw;  // {flat, q}
  uint8_t *ws;
  float *halo_a, *halo_b;
  int64_t N, N256, esc_cap;
  int Ca, keep_head, C, n_mt, n_nt, vocab, T;
  int32_t *status;
};

// r = fp32(d / step) from the reciprocal and one fused correction
__device__ __forceinline__ float div_step(float d, float step, float inv) {
  const float q0 = d * inv;
  const float e = fmaf(-q0, step, d);
  return fmaf(e, inv, q0);
}

__device__ __forceinline__ uint32_t quant_one(float d, float step, float inv, int64_t j, int r, const QuantP &P,
                                              bool &bad, float &qf) {
  if (!isfinite(d)) {
    bad = true;
    qf = 0.f;
    return 127u;
  }
  qf = fminf(fmaxf(rintf(div_step(d, step, inv)), -kQLimit), kQLimit);
  const int qi = (int)qf;
  if (qi >= -127 && qi <= 127) return (uint32_t)(qi + 127);
  Ctrl *ct = reinterpret_cast<Ctrl *>(P.ws);
  const uint32_t idx = atomicAdd(&ct->n_esc, 1u);
  if ((int64_t)idx < P.esc_cap) {
    P.esc_raw[2 * idx] = (uint32_t)(j * P.Ca + r);
    P.esc_raw[2 * idx + 1] = (uint32_t)qi;
  }
  return (uint32_t)kEsc;
}

// A buffer resource over [p, p + bytes) with a wave-uniform base: loads past
// the end return 0 and stores past it are dropped.
__device__ __forceinline__ rsrc_t span_rsrc(const void *p, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(p);
  const uint64_t bu = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b) |
                      ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(bu), (short)0,
                                           __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000);
}

// Meet the other waves once this wave's LDS accesses are done; vector memory
// operations stay in flight (s_waitcnt: vmcnt 63, expcnt 7, lgkmcnt 0).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// four integer-valued floats in [0, 255] -> the bytes of one word
__device__ __forceinline__ uint32_t pack_u8x4(float a, float b, float c, float d) {
  uint32_t w = __builtin_amdgcn_cvt_pk_u8_f32(a, 0, 0u);
  w = __builtin_amdgcn_cvt_pk_u8_f32(b, 1, w);
  w = __builtin_amdgcn_cvt_pk_u8_f32(c, 2, w);
  return __builtin_amdgcn_cvt_pk_u8_f32(d, 3, w);
}

// kKeys: the key heads come from P.keys (encode of a post-RoPE cache).  One
// launch covers the tiles of up to kLaunchBatch requests; a request's tile
// count is padded to a multiple of 8 so that its tiles keep the XCD order of
// tile_of() (the padding workgroups return at once).
template <bool kKeys>
__global__ __launch_bounds__(kThreads, 1) void k_analysis_quant(const Batch<QuantP> Bt) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int ri = batch_req(Bt, blockIdx.x);
  const QuantP &P = Bt.r[ri];
  const int local = (int)(blockIdx.x - Bt.start[ri]);
  if (local >= P.n_mt * P.n_nt) return;
  if (wg_stop(P.status)) return;
  int mt, nt;
  tile_of(local, P.n_mt * P.n_nt, P.n_nt, mt, nt);
  const int64_t m0 = (int64_t)mt * kBM;
  const int n0 = nt * kBN;
  Operand A, B;
  if (kKeys)
    set_sources(A, P.keys, kKeyCols * 2, P.rows, kD * 2, 0);
  else
    set_sources(A, P.rows, kD * 2, P.rows, kD * 2, kD / kBK);
  set_sources(B, P.A, kD * 2, P.A, kD * 2, kD / kBK);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t j = min<int64_t>(m0 + staged_row(i), P.N - 1);
    A.row[i] = (uint32_t)(P.keep_head + j);
    B.row[i] = (uint32_t)P.act[n0 + staged_row(i)];
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int N = (int)P.N;
  const int wrow0 = (int)m0 + wm * 128;  // first row of this wave's tile
  // Loaded before the main loop, whose duration hides their latency: the
  // token ids of the wave's 128 rows (rows lane and 64 + lane; rows past the
  // request read 0) and the quantiser constants of the lane's four columns.
  uint32_t tk[2];
  {
    const int l0 = threadIdx.x & 63;
    const rsrc_t tr = span_rsrc(P.tok + P.keep_head, (uint32_t)(P.T - P.keep_head) * 4u);
#pragma unroll
    for (int i = 0; i < 2; ++i) tk[i] = __builtin_amdgcn_raw_buffer_load_b32(tr, (uint32_t)(wrow0 + 64 * i + l0) * 4u, 0, 0);
  }
  f32x4 qc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
    qc[nb] = gload(reinterpret_cast<const f32x4 *>(P.qcol) + n0 + wn * 128 + nb * 32 + (threadIdx.x & 31));
  f32x16 acc[4][4];
  mainloop<true, 0, kKeys>(A, B, kD / kBK, acc, lds);

  // The epilogue works one 32x32 accumulator block at a time.  Each value
  // first takes a short path that assumes a coded row, an active rank, a
  // finite difference and no escape; a block where any of that fails (rare)
  // is decided again in full.  The means of a block are loaded six blocks
  // ahead, straight from the table into registers.  The even rows' symbols
  // wait in registers for pass 2, which writes whole symbol words.
  const int lane = epilogue_lane();
  Ctrl *ct = reinterpret_cast<Ctrl *>(P.ws);
  // LDS after the main loop: per wave, the token ids of its rows ordered
  // [lane / 32][mb][parity][e] (the 8 rows of one parity of a block row and
  // lane half, register 2e + parity, are 32 contiguous bytes), then the even
  // rows' yhat of its 16 blocks [block][e / 4][lane] (16 bytes each)
  int32_t *ltok = reinterpret_cast<int32_t *>(lds) + wave * 128;
  f32x4 *lyh = reinterpret_cast<f32x4 *>(lds + 4 * 512) + wave * 16 * 2 * 64;
  static_assert(4 * 512 + 4 * 16 * 2 * 64 * 16 <= kQuantEpiBytes, "epilogue LDS must not overlap the exchange area");
  {
    uint32_t tmax = 0u;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int R = 64 * i + lane;  // wave row: mb = R / 32, quad row q, half h, kk
      const int mb = R >> 5, q = (R >> 3) & 3, h = (R >> 2) & 1, kk = R & 3;
      ltok[((h * 4 + mb) * 2 + (kk & 1)) * 8 + 2 * q + (kk >> 1)] = (int32_t)tk[i];
      // token ids of coded rows must be in range (the table reads of any id
      // stay inside the table's buffer range)
      tmax = max(tmax, wrow0 + R < N ? tk[i] : 0u);
    }
    if (tmax >= (uint32_t)P.vocab) set_status(P.status, DCKV_EINVAL);
  }
  const rsrc_t mr = span_rsrc(P.mtab, (uint32_t)P.vocab * (uint32_t)(kC * 4));
  const uint32_t colb = (uint32_t)(n0 + wn * 128 + (lane & 31)) * 4u;
  // block row br = 4 parity + mb (0..7); its tokens are read from LDS two
  // block rows before it (at least two blocks before its first means are
  // requested, kAhead blocks before they are used)
  int tq[2][8];
  auto read_tok = [&](int br) {
    const int4 *src = reinterpret_cast<const int4 *>(ltok + (((lane >> 5) * 4 + (br & 3)) * 2 + (br >> 2)) * 8);
    const int4 t0 = src[0], t1 = src[1];
    int *d = tq[br & 1];
    d[0] = t0.x; d[1] = t0.y; d[2] = t0.z; d[3] = t0.w;
    d[4] = t1.x; d[5] = t1.y; d[6] = t1.z; d[7] = t1.w;
  };
  constexpr int kAhead = 6;
  float mq[kAhead][8];
  // means of block k of the 32 in epilogue order (block row k / 4, nb = k % 4)
  auto issue = [&](int k) {
    const int nb = k & 3;
    const int *t = tq[(k >> 2) & 1];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      mq[k % kAhead][e] = __uint_as_float(
          __builtin_amdgcn_raw_buffer_load_b32(mr, ((uint32_t)t[e] << 13) + colb + nb * 128, 0, 0));
  };
  static_assert(kC * 4 == 1 << 13, "table row bytes");
  read_tok(0);
  read_tok(1);
#pragma unroll
  for (int k = 0; k < kAhead; ++k) issue(k);

  uint32_t nonfin = 0u;  // 1 once a coded value's difference is not finite
  const uint32_t esc_cap = (uint32_t)min<int64_t>(P.esc_cap, 0x7FFFFFFF);
  // escape records of the values of one parity of a block (bit e: register 2e + par)
  auto escapes = [&](uint32_t em, const int (&qi)[8], int par, int mb, int r) {
    const int ln = epilogue_lane();
    uint32_t idx = atomicAdd(&ct->n_esc, (uint32_t)__builtin_popcount(em));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (em & (1u << e)) {
        const uint32_t j = (uint32_t)(wrow0 + acc_row(mb, 2 * e + par, ln));
        if (idx < esc_cap) {
          P.esc_raw[2 * idx] = j * (uint32_t)P.Ca + (uint32_t)r;
          P.esc_raw[2 * idx + 1] = (uint32_t)qi[e];
        }
        ++idx;
      }
    }
  };

  // pass 1: even rows, mu = H E[tok]; yhat to LDS, symbols kept for pass 2
  uint32_t ev[4][4][2];  // [mb][nb][g / 2]: byte 2 (g % 2) + i = symbol of row 4g + 2i
  float *xch = reinterpret_cast<float *>(lds + kXchOff);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const bool edge = wrow0 + mb * 32 + 32 > N;  // rows past N in this block row
    read_tok(mb + 2);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int k = mb * 4 + nb;
      const float st = qc[nb].x, inv = qc[nb].y;
      float x[8], m[8], f[8], yh[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) m[e] = mq[k % kAhead][e];
      if (k + kAhead < 32) issue(k + kAhead);  // into the slot just read
      float dsum = 0.f, amax = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = acc_get(acc[mb][nb], 2 * e);
        const float d = x[e] - m[e];
        dsum += d;
        const float qf = rintf(div_step(d, st, inv));
        amax = fmaxf(amax, fabsf(qf));
        yh[e] = m[e] + qf * st;
        f[e] = qf + 127.f;
      }
      if (edge || !(amax < 127.5f) || !isfinite(dsum)) {
        const int r = n0 + wn * 128 + nb * 32 + (lane & 31);
        int qi[8];
        uint32_t em = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const bool valid = r < P.Ca && wrow0 + acc_row(mb, 2 * e, lane) < N;
          const float d = x[e] - m[e];
          if (valid && !isfinite(d)) nonfin = 1u;
          const float qf = fminf(fmaxf(rintf(div_step(d, st, inv)), -kQLimit), kQLimit);
          qi[e] = (int)qf;
          const bool esc = valid && (qi[e] > 127 || qi[e] < -127);
          em |= (uint32_t)esc << e;
          f[e] = valid && !esc ? qf + 127.f : 255.f;
          yh[e] = valid ? m[e] + qf * st : 0.f;  // a missing right neighbour counts as zero
        }
        if (em) escapes(em, qi, 0, mb, r);
      }
      ev[mb][nb][0] = pack_u8x4(f[0], f[1], f[2], f[3]);
      ev[mb][nb][1] = pack_u8x4(f[4], f[5], f[6], f[7]);
      lyh[(k * 2) * 64 + lane] = f32x4{yh[0], yh[1], yh[2], yh[3]};
      lyh[(k * 2 + 1) * 64 + lane] = f32x4{yh[4], yh[5], yh[6], yh[7]};
      if (mb == 0 && lane < 32) {
        // the first row of each wave row: to the wave above (LDS) and, for
        // the tile's row 0, to the fix-up of the previous tile (global)
        const int r = n0 + wn * 128 + nb * 32 + lane;
        xch[wm * 256 + wn * 128 + nb * 32 + lane] = yh[0];
        if (wm == 0 && r < P.Ca) P.halo_b[(int64_t)mt * P.C + r] = yh[0];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  lds_barrier();
  const bool defer_last = m0 + kBM < P.N;
  // symbol words: one buffer per 64-rank group, holding the quads of rows < N
  // only (a group past C_a holds none)
  rsrc_t symr[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int grp = ((n0 + wn * 128) >> 6) + i;
    symr[i] = span_rsrc(P.sym32 + (size_t)grp * (size_t)(P.N256 / 4) * 64,
                        grp * 64 < P.Ca ? (uint32_t)((N + 3) >> 2) * 256u : 0u);
  }
  const uint32_t sbase = (uint32_t)((((wrow0 >> 2) + (lane >> 5)) * 64 + (lane & 31)) * 4);
  // pass 2: odd rows, mu = H E[tok] + a (yhat_{j-1} + yhat_{j+1})
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const bool edge = wrow0 + mb * 32 + 32 > N;
    if (mb < 2) read_tok(mb + 6);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int k = 16 + mb * 4 + nb;
      float x[8], m[8], mu[8], f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) m[e] = mq[k % kAhead][e];
      if (k + kAhead < 32) issue(k + kAhead);  // into the slot just read
      const f32x4 ya = lyh[((k - 16) * 2) * 64 + lane], yb = lyh[((k - 16) * 2 + 1) * 64 + lane];
      const float yv[8] = {ya.x, ya.y, ya.z, ya.w, yb.x, yb.y, yb.z, yb.w};  // yhat of register 2e
      const float st = qc[nb].x, inv = qc[nb].y, a = qc[nb].z;
      const float ext = wm == 0 && mb == 3 ? xch[256 + wn * 128 + nb * 32 + (lane & 31)] : 0.f;
      const float nx0 = mb < 3 ? lyh[((k - 12) * 2) * 64 + lane].x : 0.f;  // the next block's first row
      // the tile's last odd row (register 15 of lanes >= 32 in the last
      // block row of the lower wave) waits for the next tile's first row
      const bool dfr = mb == 3 && wm == 1 && defer_last;
      const bool dlane = dfr && lane >= 32;
      float dsum = 0.f, amax = 0.f, y2_last = 0.f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float y0 = yv[2 * g], y2 = yv[2 * g + 1];
        // the first row of the next quad: lanes < 32 hold it in lane + 32
        // (same group), lanes >= 32 in lane - 32 (next group or next block)
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(y0),
                                                         __float_as_uint(g < 3 ? yv[2 * g + 2] : nx0), false, false);
        float next3 = __uint_as_float(lane < 32 ? sw[1] : sw[0]);
        if (g == 3 && mb == 3 && lane >= 32) next3 = ext;
        if (g == 3) y2_last = y2;
        x[2 * g] = acc_get(acc[mb][nb], 4 * g + 1);
        x[2 * g + 1] = acc_get(acc[mb][nb], 4 * g + 3);
        mu[2 * g] = m[2 * g] + a * (y0 + y2);
        mu[2 * g + 1] = m[2 * g + 1] + a * (y2 + next3);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int e = 2 * g + i;
          const float d = x[e] - mu[e];
          dsum += d;
          const float qf = rintf(div_step(d, st, inv));
          amax = fmaxf(amax, e == 7 && dlane ? 0.f : fabsf(qf));
          f[e] = qf + 127.f;
        }
      }
      const int r = n0 + wn * 128 + nb * 32 + (lane & 31);
      if (edge || !(amax < 127.5f) || !isfinite(dsum)) {
        int qi[8];
        uint32_t em = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const bool valid = r < P.Ca && wrow0 + acc_row(mb, 2 * e + 1, lane) < N;
          const bool deferred = e == 7 && dlane;  // decided by the fix-up
          const float d = x[e] - mu[e];
          if (valid && !deferred && !isfinite(d)) nonfin = 1u;
          const float qf = fminf(fmaxf(rintf(div_step(d, st, inv)), -kQLimit), kQLimit);
          qi[e] = (int)qf;
          const bool esc = valid && !deferred && (qi[e] > 127 || qi[e] < -127);
          em |= (uint32_t)esc << e;
          f[e] = valid && !esc ? qf + 127.f : 255.f;
        }
        if (em) escapes(em, qi, 1, mb, r);
      }
      if (dlane) {
        f[7] = 0.f;  // finished by the fix-up
        if (r < P.Ca) P.halo_a[(int64_t)mt * P.C + r] = x[7] - m[7] - a * y2_last;
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint32_t o = __builtin_amdgcn_cvt_pk_u8_f32(f[2 * g], 1, 0u);
        o = __builtin_amdgcn_cvt_pk_u8_f32(f[2 * g + 1], 3, o);
        const uint32_t w = __builtin_amdgcn_perm(ev[mb][nb][g >> 1], o, (g & 1) ? 0x03070106u : 0x03050104u);
        __builtin_amdgcn_raw_buffer_store_b32(w, symr[nb >> 1], sbase + (uint32_t)((nb & 1) * 128 + mb * 2048 + g * 512),
                                              0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (nonfin) set_status(P.status, DCKV_EINVAL);
}


// last odd row of every row tile whose right neighbour is in the next tile
__global__ void k_encode_fixup(const Batch<QuantP> Bt) {
  const int ri = batch_req(Bt, blockIdx.x);
  const QuantP &P = Bt.r[ri];
  if (*P.status != 0) return;
  const int64_t n_fix = (P.N - 1) / kBM;  // tiles t with (t + 1) BM < N
  const int64_t i = (int64_t)(blockIdx.x - Bt.start[ri]) * blockDim.x + threadIdx.x;
  if (i >= n_fix * P.Ca) return;
  const int64_t mt = i / P.Ca;
  const int r = (int)(i - mt * P.Ca);
  const int64_t j = (mt + 1) * kBM - 1;
  const int c = P.act[r];
  const float step = P.step[c], a = P.nbr[c];
  const float d = P.halo_a[mt * P.C + r] - a * P.halo_b[(mt + 1) * P.C + r];
  bool bad = false;
  float qf;
  const uint32_t s = quant_one(d, step, 1.0f / step, j, r, P, bad, qf);
  uint8_t *sym8 = reinterpret_cast<uint8_t *>(P.sym32);
  sym8[(((size_t)(r >> 6) * (P.N256 / 4) + (j >> 2)) * 64 + (r & 63)) * 4 + (j & 3)] = (uint8_t)s;
  if (bad) set_status(P.status, DCKV_EINVAL);
}

// ---------------------------------------------------------------------------
// decode: two dequantisation passes, streamed (no GEMM: the means come from
// the plan's table)
// ---------------------------------------------------------------------------
struct DeqP {
  const float *mtab;          // [vocab][kC] embedding means
  const int32_t *tok, *rank, *colpos;
  const float *step, *nbr;
  const uint32_t *sym32;      // [G][N256/4][64]: symbols of 4 consecutive rows per word
  const uint8_t *stream;      // escape records {flat, q}, ascending flat, at the offset the parser found
  const uint8_t *ws;
  const uint32_t *esc_rows;   // [256-row tiles][2]: index range of each tile's records
  uint16_t *yhat_b;           // [NM][kC]
  int64_t N, N256;
  int Ca, keep_head, vocab;
  int32_t *status;
};

constexpr int kDeqThreads = 256;
constexpr int kDeqRows = 8;  // rows per thread: two quads (row quads share a symbol word)


// The code of escaped position (j, rank r): binary search of its flat index
// among the escape records of its 256-row tile (found by the parser).
__device__ __forceinline__ int esc_search(const DeqP &P, int j, int r) {
  const uint32_t flat = (uint32_t)j * (uint32_t)P.Ca + (uint32_t)r;
  const uint32_t *rec = reinterpret_cast<const uint32_t *>(P.stream + gload(&reinterpret_cast<const Ctrl *>(P.ws)->esc_off));
  uint32_t lo = gload(P.esc_rows + 2 * (j >> 8)), hi = gload(P.esc_rows + 2 * (j >> 8) + 1);
  const uint32_t end = hi;
  while (lo < hi) {
    const uint32_t mid = (lo + hi) >> 1;
    if (gload(rec + 2 * mid) < flat) lo = mid + 1; else hi = mid;
  }
  if (lo < end && gload(rec + 2 * lo) == flat) return (int)gload(rec + 2 * lo + 1);
  set_status(P.status, DCKV_ECORRUPT);
  return 0;
}

// Thread t of grid row y owns components c0 .. c0+3 (c0 = 4 (256 y + t)) of
// rows j0 .. j0+7 (j0 = 8 x), plus the first row j0+8 of the next rows, which
// the last odd row needs.  Every load is issued up front: the 9 rows' tokens
// and means (a 16-byte load per row), and three symbol words per component
// (rows j0..j0+3, j0+4..j0+7, j0+8..).  Pass 1 gives the even rows
// (yhat = mu + q step), pass 2 the odd rows (mu += a (yhat_{j-1} +
// yhat_{j+1})); rows past the end count as zero.  kDense: no dropped
// component, so component = rank = table column.
template <bool kDense>
__global__ __launch_bounds__(kDeqThreads) void k_dequant(const Batch<DeqP> Bt) {
  const int ri = batch_req(Bt, blockIdx.x);
  const DeqP &P = Bt.r[ri];
  const uint32_t local = blockIdx.x - Bt.start[ri];
  constexpr uint32_t kCols = kC / (4 * kDeqThreads);  // workgroups across a row's components
  const uint32_t by = local % kCols, bx = local / kCols;
  if (gload(P.status) != 0) return;
  const int c0 = (by * kDeqThreads + threadIdx.x) * 4;
  const int j0 = bx * kDeqRows;
  const int N = (int)P.N;
  const size_t n_quads = (size_t)(P.N256 / 4);
  float st[4], a[4];
  int r[4], col[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    st[k] = gload(P.step + c0 + k);
    a[k] = gload(P.nbr + c0 + k);
    r[k] = kDense ? c0 + k : gload(P.rank + c0 + k);
    col[k] = kDense ? c0 + k : gload(P.colpos + c0 + k);
  }
  // symbol words of the three quads (code 0 where dropped or past the end)
  uint32_t w[3][4];
#pragma unroll
  for (int qq = 0; qq < 3; ++qq) {
    const size_t q = (size_t)(j0 >> 2) + qq;
    if (j0 + 4 * qq < N) {
      if (kDense) {
        const u32x4 x = gload(reinterpret_cast<const u32x4 *>(P.sym32 + ((size_t)(c0 >> 6) * n_quads + q) * 64 + (c0 & 63)));
        w[qq][0] = x.x; w[qq][1] = x.y; w[qq][2] = x.z; w[qq][3] = x.w;
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          w[qq][k] = r[k] >= 0 ? gload(P.sym32 + ((size_t)(r[k] >> 6) * n_quads + q) * 64 + (r[k] & 63)) : 0x7F7F7F7Fu;
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) w[qq][k] = 0x7F7F7F7Fu;
    }
  }
  // means of the 9 rows (0 past the end)
  float m[kDeqRows + 1][4];
#pragma unroll
  for (int i = 0; i <= kDeqRows; ++i) {
    if (j0 + i < N) {
      int v = gload(P.tok + P.keep_head + j0 + i);
      if (v < 0 || v >= P.vocab) {
        set_status(P.status, DCKV_EINVAL);
        v = 0;
      }
      const float *row = P.mtab + (size_t)v * kC;
      if (kDense) {
        const f32x4 x = gload(reinterpret_cast<const f32x4 *>(row + c0));
        m[i][0] = x.x; m[i][1] = x.y; m[i][2] = x.z; m[i][3] = x.w;
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) m[i][k] = gload(row + col[k]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) m[i][k] = 0.f;
    }
  }
  // codes; escaped positions (symbol 255) are looked up, one at a time
  float q[kDeqRows + 1][4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t em = 0;
#pragma unroll
    for (int i = 0; i <= kDeqRows; ++i) {
      const uint32_t sy = (w[i >> 2][k] >> (8 * (i & 3))) & 0xFFu;
      q[i][k] = (float)((int)sy - 127);
      if (sy == (uint32_t)kEsc && j0 + i < N) em |= 1u << i;
    }
    while (em) {
      const int i = __builtin_ctz(em);
      em &= em - 1;
      const float val = (float)esc_search(P, j0 + i, r[k]);
#pragma unroll
      for (int ii = 0; ii <= kDeqRows; ++ii)
        if (ii == i) q[ii][k] = val;
    }
  }
  // pass 1: even rows (row j0+8 too); pass 2: odd rows
  float y[kDeqRows + 1][4];
#pragma unroll
  for (int i = 0; i <= kDeqRows; i += 2)
#pragma unroll
    for (int k = 0; k < 4; ++k) y[i][k] = j0 + i < N ? m[i][k] + q[i][k] * st[k] : 0.f;
#pragma unroll
  for (int i = 1; i < kDeqRows; i += 2)
#pragma unroll
    for (int k = 0; k < 4; ++k) y[i][k] = m[i][k] + a[k] * (y[i - 1][k] + y[i + 1][k]) + q[i][k] * st[k];
#pragma unroll
  for (int i = 0; i < kDeqRows; ++i) {
    if (j0 + i < N) {
      u32x2 o;
      o.x = pack_bf16x2(y[i][0], y[i][1]);
      o.y = pack_bf16x2(y[i][2], y[i][3]);
      *(u32x2 __attribute__((address_space(1))) *)(P.yhat_b + (size_t)(j0 + i) * kC + c0) = o;
    }
  }
}


// Where decoded rows go: rows [T][D] (rows set) or the per-layer head
// matrices (heads[2 l + kv] -> [2][T][head_dim]).
struct OutRows {
  uint16_t *rows;
  uint16_t *heads[12];
  int64_t T;
  // element (position pos, head, 0) of the output
  __device__ __forceinline__ uint16_t *at(int64_t pos, int head) const {
    return rows ? rows + (size_t)pos * kD + head * kHeadDim
                : heads[head >> 1] + ((size_t)(head & 1) * T + pos) * kHeadDim;
  }
};

static OutRows out_rows(const DecodeArgs &a) {
  OutRows o{};
  o.T = a.g.T;
  if (a.heads) {
    o.rows = nullptr;
    for (int i = 0; i < 12; ++i) o.heads[i] = a.heads->p[i];
  } else {
    o.rows = a.rows_out;
  }
  return o;
}

// kept row k: RoPE on the key columns of the verbatim row in the stream.
// Thread t takes the pair (d, d + 128), d = t % 128, of heads 2 j + t / 128,
// j < 24 / 2 (even j: a layer's key heads, odd j: its value heads); every load
// is issued before the first store.  256 threads.
constexpr int kKeptThreads = 256;
__device__ __forceinline__ void kept_rope_row(int64_t k, const uint8_t *stream, const float2 *lo, const float2 *hi,
                                              const OutRows &out, int64_t head_n, int64_t tail_pos0) {
  constexpr int kJ = kD / 2 / kKeptThreads;
  static_assert(kD / 2 % kKeptThreads == 0 && kKeptThreads == 2 * kHalf, "kept-row thread layout");
  const int64_t pos = k < head_n ? k : tail_pos0 + (k - head_n);
  const uint16_t *src = reinterpret_cast<const uint16_t *>(stream + kHeaderBytes) + (size_t)k * kD;
  const int d = threadIdx.x & (kHalf - 1), hsub = threadIdx.x >> 7;
  uint16_t x0[kJ], x1[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const int base = (2 * j + hsub) * kHeadDim;
    x0[j] = src[base + d];
    x1[j] = src[base + d + kHalf];
  }
  // the angle pos * w_d, the same for every key head
  const float2 a = lo[(size_t)(pos & 255) * kHalf + d], b = hi[(size_t)(pos >> 8) * kHalf + d];
  const float cs = b.x * a.x - b.y * a.y;
  const float sn = b.y * a.x + b.x * a.y;
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    uint16_t *dst = out.at(pos, 2 * j + hsub);
    if ((j & 1) == 0) {
      const float v0 = bf2f(x0[j]), v1 = bf2f(x1[j]);
      dst[d] = f2bf(v0 * cs - v1 * sn);
      dst[d + kHalf] = f2bf(v1 * cs + v0 * sn);
    } else {
      dst[d] = x0[j];
      dst[d + kHalf] = x1[j];
    }
  }
}

// ---------------------------------------------------------------------------
// decode: correction hidden layer h = GELU(W1 yhat_b)
// ---------------------------------------------------------------------------
struct W1P {
  const uint16_t *yhat_b, *W1;
  float *part;       // [2][NM][256]: the products over each half of the coefficients
  uint16_t *h_b;     // [NM][256]
  int64_t N, NM;
  int n_mt;
  int32_t *status;
  // kept rows, RoPE'd by the GELU kernel's first n_kept workgroups
  const uint8_t *stream;
  const float2 *rope_lo, *rope_hi;
  OutRows out;
  int64_t n_kept, head_n, tail_pos0;
};

// W1 yhat_b as two half-K products (coefficients [0, 1024) and [1024, 2048)):
// 256-row tiles times 2 halves fill twice as many CUs as whole-K tiles; the
// halves are added (one fp32 addition, so the order does not matter) by
// k_w1_gelu.
constexpr int kW1Batch = kLaunchBatch;  // requests per launch of the W1 kernels
static_assert(sizeof(Batch<W1P, kW1Batch>) <= 4096, "kernel argument size");

__global__ __launch_bounds__(kThreads, 1) void k_w1(const Batch<W1P, kW1Batch> Bt) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int ri = batch_req(Bt, blockIdx.x);
  const W1P &P = Bt.r[ri];
  const uint32_t local = blockIdx.x - Bt.start[ri];
  if (wg_stop(P.status)) return;
  int mt, kh;
  tile_of((int)local, P.n_mt * 2, 2, mt, kh);
  const int64_t m0 = (int64_t)mt * kBM;
  Operand A, B;
  set_sources(A, P.yhat_b + kh * (kC / 2), kC * 2, P.yhat_b + kh * (kC / 2), kC * 2, kC / 2 / kBK);
  set_sources(B, P.W1 + kh * (kC / 2), kC * 2, P.W1 + kh * (kC / 2), kC * 2, kC / 2 / kBK);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    A.row[i] = (uint32_t)(m0 + staged_row(i));
    B.row[i] = (uint32_t)staged_row(i);
  }
  f32x16 acc[4][4];
  mainloop(A, B, kC / 2 / kBK, acc, lds);
  const int lane = epilogue_lane(), wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  float *part = P.part + ((size_t)kh * P.NM + m0 + wm * 128) * kHid + wn * 128 + (lane & 31);
  const int rows_left = (int)min<int64_t>(P.N - (m0 + wm * 128), 128);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const f32x16 b = acc_block(acc, mb, nb);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = acc_row(mb, v, lane);
        if (row < rows_left) part[(size_t)row * kHid + nb * 32] = b[v];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
}

// h_b = bf16(GELU(part0 + part1)), exact-erf GELU; 4 hidden units per thread.
// The first n_kept workgroups apply RoPE to one kept row each (the RoPE tables
// are written by the parse kernel, which runs first); they come first so that
// their loads overlap the GELU workgroups rather than trail them.
__global__ __launch_bounds__(kKeptThreads) void k_w1_gelu(const Batch<W1P, kW1Batch> Bt) {
  const int ri = batch_req(Bt, blockIdx.x);
  const W1P &P = Bt.r[ri];
  const uint32_t local = blockIdx.x - Bt.start[ri];
  if (*P.status != 0) return;
  if (local < P.n_kept) {
    kept_rope_row(local, P.stream, P.rope_lo, P.rope_hi, P.out, P.head_n, P.tail_pos0);
    return;
  }
  const int64_t i = (int64_t)(local - P.n_kept) * blockDim.x + threadIdx.x;  // (row, 4-unit group)
  if (i >= P.N * (kHid / 4)) return;
  const size_t o = (size_t)i * 4;
  const f32x4 a = *reinterpret_cast<const f32x4 *>(P.part + o);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(P.part + (size_t)P.NM * kHid + o);
  float h[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float u = a[k] + b[k];
    h[k] = 0.5f * u * (1.0f + erff(u * 0.70710678118654752f));
  }
  u32x2 w;
  w.x = pack_bf16x2(h[0], h[1]);
  w.y = pack_bf16x2(h[2], h[3]);
  *reinterpret_cast<u32x2 *>(P.h_b + o) = w;
}

// ---------------------------------------------------------------------------
// decode: synthesis xhat = S yhat_b + W2 h_b with RoPE on key heads
// ---------------------------------------------------------------------------
struct SynP {
  const uint16_t *yhat_b, *h_b, *S, *W2;
  const float2 *rope_lo, *rope_hi;  // [256][128], [ceil(T/256)][128]: (cos, sin)
  OutRows out;
  int64_t N;
  int keep_head, n_mt, n_nt;
  int32_t *status;
};

// Tile nt covers head nt (256 dims).  Wave column half wn, block nb < 2 holds
// dims 64 wn + 32 nb + [0, 32); block nb + 2 holds the same dims + 128, so a
// rotate-half pair (d, d + 128) is one lane's register v of blocks nb, nb + 2.
__device__ __forceinline__ int syn_dim(int n) {
  const int wn = n >> 7, nb = (n >> 5) & 3, j = n & 31;
  return (nb >> 1) * 128 + 64 * wn + 32 * (nb & 1) + j;
}

// Rows r, r + 1 of this lane's column j (y0, y1) -> one word of a row and two
// adjacent columns: lanes l and l ^ 1 (columns j, j ^ 1) swap their packed
// pairs with a DPP quad permute; the even lane keeps row r (columns j, j + 1),
// the odd lane row r + 1 (columns j - 1, j).  sel is the lane's v_perm
// selector (0x05040100 on even lanes, 0x03020706 on odd ones).
__device__ __forceinline__ uint32_t row_pair_word(float y0, float y1, uint32_t sel) {
  const uint32_t pk = pack_bf16x2(y0, y1);
  const uint32_t sw = (uint32_t)__builtin_amdgcn_mov_dpp((int)pk, 0xB1, 0xF, 0xF, false);
  return __builtin_amdgcn_perm(sw, pk, sel);
}

// Word p of a wave's packed output tile: p = ((mb 4 + nb) 4 + g) 2 + h holds
// tile row acc_crow(mb, 4g + 2h) + 4 (lane / 32) + lane % 2 and the columns
// (lane % 32) & ~1 and + 1 of block nb.  Its byte offset from the wave's
// origin (row 0, first column of the wave's half of the head), without the
// lane's part; block nb holds head dims (nb / 2) 128 + 32 (nb % 2) + [0, 32).
template <int kLd>  // row stride of the output (kD for rows, kHeadDim for head matrices)
__device__ __forceinline__ constexpr uint32_t pend_off(int p) {
  return (uint32_t)((acc_crow(p >> 5, 4 * ((p >> 1) & 3) + 2 * (p & 1)) * kLd + ((p >> 3) & 3) / 2 * 128 +
                     32 * (((p >> 3) & 3) & 1)) * 2);
}

// Persistent: each workgroup takes tiles b, b + grid, ...  Of the 128 x 128
// bf16 outputs of a wave (128 words per lane), kSynDefer words per lane stay
// in registers after the epilogue and are stored during the first k-tiles of
// the next tile's main loop, so that the stores of all CUs do not come at the
// same moment (the rest, as many as the registers left by the main loop do
// not hold, are stored at once); the last tile's words are stored at the end.  A buffer resource per tile ends at the
// last coded row, so stores of rows past N are dropped.
constexpr int kSynDefer = 96;             // words held over (the rest are stored at once)
constexpr int kSynPeel = kSynDefer / 8;    // k-tiles that store them, 8 each
static_assert(kC / kBK >= kSynPeel, "synthesis main loop shorter than the store spread");

// KT: k-tiles, 36 with the correction, 32 for the linear codec; kHeads: the
// per-layer head matrices as the output.  The tiles of up to kLaunchBatch
// requests form one sequence (each request's count padded to a multiple of 8,
// which keeps tile_of()'s XCD order); a tile of a request whose status is set
// is skipped, and the words held over from the tile before are still stored.
template <int KT, bool kHeads>
__global__ __launch_bounds__(kThreads, 1) void k_synthesis(const Batch<SynP> Bt) {
  constexpr int kLd = kHeads ? kHeadDim : kD;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int total = (int)Bt.start[Bt.n];
  uint32_t pend[kSynDefer];
  rsrc_t pr;          // the tile of the words
  uint32_t lb = 0u, sel = 0u;
  bool have = false;  // wave-uniform
  auto store_pend = [&](int p) {
    __builtin_amdgcn_raw_buffer_store_b32(pend[p], pr, lb + pend_off<kLd>(p), 0, 0);
  };
  // word p of this tile: held over, or stored now
  auto put = [&](int p, uint32_t w) {
    if (p < kSynDefer)
      pend[p] = w;
    else
      __builtin_amdgcn_raw_buffer_store_b32(w, pr, lb + pend_off<kLd>(p), 0, 0);
  };
#pragma unroll 1
  for (int t = blockIdx.x; t < total; t += gridDim.x) {
    const int ri = batch_req(Bt, (uint32_t)t);
    const SynP &P = Bt.r[ri];
    const int local = t - (int)Bt.start[ri];
    if (local >= P.n_mt * P.n_nt || wg_stop(P.status)) continue;
    int mt, nt;
    tile_of(local, P.n_mt * P.n_nt, P.n_nt, mt, nt);
    const int64_t m0 = (int64_t)mt * kBM;
    const int head = nt;
    Operand A, B;
    set_sources(A, P.yhat_b, kC * 2, P.h_b, kHid * 2, kC / kBK);
    set_sources(B, P.S, kC * 2, P.W2, kHid * 2, kC / kBK);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      A.row[i] = (uint32_t)(m0 + staged_row(i));
      B.row[i] = (uint32_t)(head * kHeadDim + syn_dim(staged_row(i)));
    }
    f32x16 acc[4][4];
    if (have)
      mainloop<true, kSynPeel>(A, B, KT, acc, lds, store_pend);
    else
      mainloop(A, B, KT, acc, lds);

    const int lane = epilogue_lane();
    const bool is_key = (head & 3) < 2;  // per layer: 2 key heads, then 2 value heads
    const int64_t wrow0 = m0 + wm * 128;
    // this tile's words: rows from keep_head + wrow0, columns from the
    // wave's half of the head
    {
      const int64_t r0 = P.keep_head + wrow0;
      const int64_t rows = max<int64_t>(0, P.N - wrow0);
      pr = span_rsrc(P.out.at(r0, head) + 64 * wn, (uint32_t)min<int64_t>(rows * kLd * 2, 0x7FFFFFFF));
      lb = (uint32_t)(((4 * (lane >> 5) + (lane & 1)) * kLd + ((lane & 31) & ~1)) * 2);
      sel = (lane & 1) ? 0x03020706u : 0x05040100u;
    }
    if (is_key) {
      // Angles: the lane's first row from the tables (position p = 256 hi +
      // lo), every other row by rotating it through 32 (block), 8 (register
      // group) and 1 (row) positions, whose cos / sin are rows 32, 8 and 1 of
      // the low table.  All table loads are issued before the first rotation.
      // The position of a lane whose first row is past the end is clamped
      // only to stay inside the tables (its words are dropped).
      const int64_t p0 = P.keep_head + min<int64_t>(wrow0 + 4 * (lane >> 5), P.N - 1);
      float2 ta[2], tb[2], r1[2], r8[2], r32[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int f = 64 * wn + 32 * nb + (lane & 31);  // rotary frequency index
        ta[nb] = P.rope_lo[(size_t)(p0 & 255) * kHalf + f];
        tb[nb] = P.rope_hi[(size_t)(p0 >> 8) * kHalf + f];
        r1[nb] = P.rope_lo[1 * kHalf + f];
        r8[nb] = P.rope_lo[8 * kHalf + f];
        r32[nb] = P.rope_lo[32 * kHalf + f];
      }
      auto rot = [](float &c, float &s, float2 r) {
        const float c2 = c * r.x - s * r.y;
        s = s * r.x + c * r.y;
        c = c2;
      };
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float c_mb = tb[nb].x * ta[nb].x - tb[nb].y * ta[nb].y;
        float s_mb = tb[nb].y * ta[nb].x + tb[nb].x * ta[nb].y;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          float c_g = c_mb, s_g = s_mb;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float cs = c_g, sn = s_g;
            float o0[4], o1[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int v = 4 * g + i;
              const float lo = acc_get(acc[mb][nb], v), hi = acc_get(acc[mb][nb + 2], v);
              o0[i] = lo * cs - hi * sn;
              o1[i] = hi * cs + lo * sn;
              if (i < 3) rot(cs, sn, r1[nb]);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              put(((mb * 4 + nb) * 4 + g) * 2 + h, row_pair_word(o0[2 * h], o0[2 * h + 1], sel));
              put(((mb * 4 + nb + 2) * 4 + g) * 2 + h, row_pair_word(o1[2 * h], o1[2 * h + 1], sel));
            }
            if (g < 3) rot(c_g, s_g, r8[nb]);
          }
          if (mb < 3) rot(c_mb, s_mb, r32[nb]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
          for (int q = 0; q < 8; ++q)
            put((mb * 4 + nb) * 8 + q, row_pair_word(acc_get(acc[mb][nb], 2 * q), acc_get(acc[mb][nb], 2 * q + 1), sel));
          __builtin_amdgcn_sched_barrier(0);
        }
    }
    have = true;
  }
  if (have) {
#pragma unroll
    for (int p = 0; p < kSynDefer; ++p) store_pend(p);
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <class K, class P>
static void launch_gemm(K kernel, const char *name, int grid, const P &prm, hipStream_t s) {
  // dynamic LDS above 64 KiB has to be allowed per kernel
  (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            kLdsBytes);
  KernelTimer tm(name, s);
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), kLdsBytes, s, prm);
}

static int prepare_f32(GemmF32Args &P) {
  P.n_mt = (P.M + kBM - 1) / kBM;
  P.n_nt = (P.N + kBN - 1) / kBN;
  if (P.ksplit < 1) P.ksplit = 1;
  return P.n_mt * P.n_nt * P.ksplit;
}

void launch_gemm_f32(const GemmF32Args &args, hipStream_t s) {
  GemmF32Pair PP;
  PP.g0 = args;
  PP.blocks0 = prepare_f32(PP.g0);
  PP.g1 = PP.g0;
  launch_gemm(k_gemm_f32, "fit_gemm", PP.blocks0, PP, s);
}

void launch_gemm_f32_pair(const GemmF32Args &a, const GemmF32Args &b, hipStream_t s) {
  GemmF32Pair PP;
  PP.g0 = a;
  PP.g1 = b;
  PP.blocks0 = prepare_f32(PP.g0);
  const int blocks1 = prepare_f32(PP.g1);
  launch_gemm(k_gemm_f32, "fit_gemm", PP.blocks0 + blocks1, PP, s);
}

int build_mean_table(dckv_plan_t *p) {
  MeanTabP P;
  P.E = p->E;
  P.H = p->H;
  P.perm = p->dev.perm;
  P.mtab = p->mtab;
  P.vocab = p->vocab;
  P.n_mt = (p->vocab + kBM - 1) / kBM;
  P.n_nt = kC / kBN;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev != p->device)
    return set_error(DCKV_EHIP, "plan: the current device changed while building the plan");
  (void)hipFuncSetAttribute(reinterpret_cast<const void *>(k_mean_table),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  hipLaunchKernelGGL(k_mean_table, dim3(P.n_mt * P.n_nt), dim3(kThreads), kLdsBytes, 0, P);
  int rc = check_hip(hipGetLastError(), "plan: mean table launch");
  if (rc) return rc;
  return check_hip(hipStreamSynchronize(0), "plan: mean table");
}

static QuantP quant_params(const EncodeArgs &a) {
  QuantP P;
  P.rows = a.rows;
  P.keys = a.keys;
  P.A = a.p->A;
  P.act = a.p->dev.act;
  P.tok = a.tok;
  P.step = a.p->dev.step;
  P.nbr = a.p->dev.nbr;
  P.qcol = a.p->dev.qcol;
  P.mtab = a.p->mtab;
  P.sym32 = reinterpret_cast<uint32_t *>(a.ws + a.l.sym);
  P.esc_raw = reinterpret_cast<uint32_t *>(a.ws + a.l.esc_raw);
  P.ws = a.ws;
  P.halo_a = reinterpret_cast<float *>(a.ws + a.l.halo_a);
  P.halo_b = reinterpret_cast<float *>(a.ws + a.l.halo_b);
  P.N = a.g.N;
  P.N256 = a.g.N256;
  P.esc_cap = a.g.esc_cap;
  P.Ca = a.p->C_a;
  P.keep_head = a.p->keep_head;
  P.C = a.p->C;
  P.n_mt = (int)a.g.n_mtiles;
  P.n_nt = (int)(a.g.Ca4 / kBN);
  P.vocab = a.p->vocab;
  P.T = (int)a.g.T;
  P.status = a.status;
  return P;
}

// a launch's parameters stay within the 4 KiB of kernel arguments
static_assert(sizeof(Batch<QuantP>) <= 4096 && sizeof(Batch<SynP>) <= 4096, "kernel argument size");

// tiles of one request's GEMM, padded to a multiple of 8 (see k_analysis_quant)
static uint32_t padded_tiles(int64_t n_mt, int64_t n_nt) { return (uint32_t)((n_mt * n_nt + 7) / 8 * 8); }

void launch_analysis_gemm(const EncodeArgs *args, int n) {
  // requests with a key copy (post-RoPE encode) take the other variant
  for (int keys = 0; keys < 2; ++keys) {
    std::vector<int> idx;
    for (int i = 0; i < n; ++i)
      if ((args[i].keys != nullptr) == (keys == 1) && args[i].g.N > 0 && args[i].p->C_a > 0) idx.push_back(i);
    if (idx.empty()) continue;
    auto fill = [&](int k) { return quant_params(args[idx[k]]); };
    auto count = [&](int k) {
      const QuantP P = quant_params(args[idx[k]]);
      return padded_tiles(P.n_mt, P.n_nt);
    };
    if (keys)
      launch_batched<QuantP>(k_analysis_quant<true>, "analysis_gemm", (int)idx.size(), args[0].s, kThreads, fill,
                             count, kLdsBytes);
    else
      launch_batched<QuantP>(k_analysis_quant<false>, "analysis_gemm", (int)idx.size(), args[0].s, kThreads, fill,
                             count, kLdsBytes);
  }
}

void launch_encode_fixup(const EncodeArgs *args, int n) {
  auto fill = [&](int i) { return quant_params(args[i]); };
  auto count = [&](int i) {
    const EncodeArgs &a = args[i];
    if (a.g.N == 0 || a.p->C_a == 0) return 0u;
    const int64_t n_fix = (a.g.N - 1) / kBM;  // tiles t with (t+1)*BM < N
    return n_fix <= 0 ? 0u : (uint32_t)((n_fix * a.p->C_a + 255) / 256);
  };
  launch_batched<QuantP>(k_encode_fixup, "fixup", n, args[0].s, 256, fill, count);
}

void launch_dequant(const DecodeArgs *args, int n) {
  auto fill = [&](int i) {
    const DecodeArgs &a = args[i];
    DeqP P;
    P.mtab = a.p->mtab;
    P.tok = a.tok;
    P.rank = a.p->dev.rank;
    P.colpos = a.p->dev.colpos;
    P.step = a.p->dev.step;
    P.nbr = a.p->dev.nbr;
    P.sym32 = reinterpret_cast<const uint32_t *>(a.ws + a.l.sym);
    P.stream = a.stream;
    P.ws = a.ws;
    P.esc_rows = reinterpret_cast<const uint32_t *>(a.ws + a.l.esc_rows);
    P.yhat_b = reinterpret_cast<uint16_t *>(a.ws + a.l.yhat_b);
    P.N = a.g.N;
    P.N256 = a.g.N256;
    P.Ca = a.p->C_a;
    P.keep_head = a.p->keep_head;
    P.vocab = a.p->vocab;
    P.status = a.status;
    return P;
  };
  // requests whose rANS decode dequantised them already are skipped; the
  // others without dropped components take the dense variant; the others
  // (in their own launches) read symbols and means through rank and colpos
  for (int dense = 1; dense >= 0; --dense) {
    std::vector<int> idx;
    for (int i = 0; i < n; ++i)
      if (args[i].g.N > 0 && (args[i].p->C_a == kC) == (dense == 1) && !dequant_fused(args[i])) idx.push_back(i);
    if (idx.empty()) continue;
    auto f = [&](int k) { return fill(idx[k]); };
    auto count = [&](int k) {
      const DecodeArgs &a = args[idx[k]];
      return (uint32_t)(((a.g.N + kDeqRows - 1) / kDeqRows) * (kC / (4 * kDeqThreads)));
    };
    if (dense)
      launch_batched<DeqP>(k_dequant<true>, "dequant", (int)idx.size(), args[0].s, kDeqThreads, f, count);
    else
      launch_batched<DeqP>(k_dequant<false>, "dequant", (int)idx.size(), args[0].s, kDeqThreads, f, count);
  }
}

void launch_w1_gemm(const DecodeArgs *args, int n) {
  auto fill = [&](int i) {
    const DecodeArgs &a = args[i];
    W1P P;
    P.yhat_b = reinterpret_cast<const uint16_t *>(a.ws + a.l.yhat_b);
    P.W1 = a.p->W1;
    P.part = reinterpret_cast<float *>(a.ws + a.l.w1_part);
    P.h_b = reinterpret_cast<uint16_t *>(a.ws + a.l.h_b);
    P.N = a.g.N;
    P.NM = a.g.NM;
    P.n_mt = (int)a.g.n_mtiles;
    P.status = a.status;
    P.stream = a.stream;
    P.rope_lo = reinterpret_cast<const float2 *>(a.ws + a.l.rope_lo);
    P.rope_hi = reinterpret_cast<const float2 *>(a.ws + a.l.rope_hi);
    P.out = out_rows(a);
    P.n_kept = a.g.n_kept;
    P.head_n = std::min<int64_t>(a.p->keep_head, a.g.T);
    P.tail_pos0 = a.p->keep_head + a.g.N;
    return P;
  };
  auto gemm_count = [&](int i) {
    const DecodeArgs &a = args[i];
    return (a.g.N && a.p->W1) ? (uint32_t)(a.g.n_mtiles * 2) : 0u;
  };
  launch_batched<W1P, kW1Batch>(k_w1, "w1_gemm", n, args[0].s, kThreads, fill, gemm_count, kLdsBytes);
  // the linear codec (no correction) launches the kept rows only
  auto gelu_count = [&](int i) {
    const DecodeArgs &a = args[i];
    const unsigned gb = a.p->W1 ? (unsigned)((a.g.N * (kHid / 4) + 255) / 256) : 0u;
    return gb + (uint32_t)a.g.n_kept;
  };
  launch_batched<W1P, kW1Batch>(k_w1_gelu, "w1_gelu", n, args[0].s, kKeptThreads, fill, gelu_count);
}

static SynP syn_params(const DecodeArgs &a) {
  SynP P;
  P.yhat_b = reinterpret_cast<const uint16_t *>(a.ws + a.l.yhat_b);
  P.h_b = reinterpret_cast<const uint16_t *>(a.ws + a.l.h_b);
  P.S = a.p->S;
  P.W2 = a.p->W2;
  P.rope_lo = reinterpret_cast<const float2 *>(a.ws + a.l.rope_lo);
  P.rope_hi = reinterpret_cast<const float2 *>(a.ws + a.l.rope_hi);
  P.out = out_rows(a);
  P.N = a.g.N;
  P.keep_head = a.p->keep_head;
  P.n_mt = (int)a.g.n_mtiles;
  P.n_nt = kD / kBN;
  P.status = a.status;
  return P;
}

void launch_synthesis_gemm(const DecodeArgs *args, int n) {
  // persistent: one workgroup per CU at most
  static int n_cu = 0;
  if (n_cu == 0) {
    int dev = 0, c = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0)
      n_cu = c;
    else
      n_cu = 256;
  }
  constexpr int kFull = (kC + kHid) / kBK, kLin = kC / kBK;
  // one sequence of launches per kernel variant: correction or linear codec,
  // rows or head matrices
  for (int var = 0; var < 4; ++var) {
    const bool lin = var & 1, heads = var >> 1;
    std::vector<int> idx;
    for (int i = 0; i < n; ++i)
      if (args[i].g.N > 0 && (args[i].p->W1 == nullptr) == lin && (args[i].heads != nullptr) == heads)
        idx.push_back(i);
    for (size_t i0 = 0; i0 < idx.size(); i0 += kLaunchBatch) {
      Batch<SynP> B{};
      B.n = (int)std::min<size_t>(kLaunchBatch, idx.size() - i0);
      uint32_t w = 0;
      for (int r = 0; r < B.n; ++r) {
        B.start[r] = w;
        B.r[r] = syn_params(args[idx[i0 + r]]);
        w += padded_tiles(B.r[r].n_mt, B.r[r].n_nt);
      }
      for (int r = B.n; r <= kLaunchBatch; ++r) B.start[r] = w;
      const int grid = std::min<int>((int)w, n_cu);
      if (heads) {
        if (lin)
          launch_gemm(k_synthesis<kLin, true>, "synthesis_gemm", grid, B, args[0].s);
        else
          launch_gemm(k_synthesis<kFull, true>, "synthesis_gemm", grid, B, args[0].s);
      } else {
        if (lin)
          launch_gemm(k_synthesis<kLin, false>, "synthesis_gemm", grid, B, args[0].s);
        else
          launch_gemm(k_synthesis<kFull, false>, "synthesis_gemm", grid, B, args[0].s);
      }
    }
  }
}

}  // namespace dckv
