// Internal declarations shared by the host runtime and the HIP kernels of the
// DCKV codec library.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/dckv.h"

namespace dckv {

// ---- fixed format and kernel constants -----------------------------------
constexpr int kPrecBits = 15;               // table precision
constexpr uint32_t kM = 1u << kPrecBits;    // 32768
constexpr uint32_t kL = 1u << 16;           // rANS lower bound
constexpr int kNSym = 255;                  // codes -127..127
constexpr int kEsc = 255;                   // escaped position marker
constexpr int kBlock = 256;                 // tokens per substream block
constexpr int kLanes = 64;                  // components per group (one wave)
constexpr int kBuckets = 256;               // decode lookup buckets per table (128 slots each)
constexpr int kBucketShift = kPrecBits - 8; // slot >> 7 -> bucket
constexpr uint32_t kSplitPure = kM;         // bucket split: one symbol (no slot reaches it)
constexpr uint32_t kSplitSearch = 0xFFFFu;  // bucket split: three or more symbols
constexpr int kHeaderBytes = 64;
constexpr uint16_t kVersion = 1;

// GEMM tiling shared by every transform kernel
constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 64;

// fixed shapes supported by the kernels
constexpr int kD = 6144;
// Positions of one request (and calibration rows of a fit): the GEMMs address
// each operand through one buffer resource with 32-bit byte offsets, so a
// [rows][6,144] bf16 operand must stay below 4 GiB; 2^18 rows is 3 GiB.
constexpr int64_t kMaxRows = (int64_t)1 << 18;
constexpr int kC = 2048;
// The encoder reads a token's row of the embedding-mean table (n_coef fp32 =
// 8 KiB) through a buffer resource with 32-bit byte offsets, so the table's
// vocab * 8 KiB must stay below 4 GiB.
constexpr int kMaxVocab = (1 << 19) - 1;
constexpr int kHid = 256;
constexpr int kEmb = 2048;
constexpr int kHeadDim = 256;
constexpr int kHalf = kHeadDim / 2;
constexpr int kKeyCols = 6 * 2 * kHeadDim;  // the key heads of a row (n_layers * n_kv_heads * head_dim)

// ---- plan ----------------------------------------------------------------
struct PlanDev {
  float *step = nullptr;        // [C]
  float *nbr = nullptr;         // [C]
  int32_t *rank = nullptr;      // [C]   rank or -1
  int32_t *act = nullptr;       // [C_a] component of each rank (padded to a kBN multiple)
  int32_t *perm = nullptr;      // [C]   component of each mean-table column: ranks, then dropped
  int32_t *colpos = nullptr;    // [C]   mean-table column of each component
  float *qcol = nullptr;        // [C_a padded][4] step, 1/step (0 past C_a), neighbour weight, 0 of each rank
  float *scale = nullptr;       // [C]   Laplace scale b of each component
  uint32_t *tab = nullptr;      // [C_a][256]  f | cum << 16
  float *rcp = nullptr;         // [C_a][256]  fp32(1/f (1 - 2^-21)), the encoder's quotient estimate
  uint32_t *bucket = nullptr;   // [C_a][kBuckets] lo | split << 16 of each slot bucket (decoder)
  double *omega = nullptr;      // [head_dim/2] RoPE frequencies
};

}  // namespace dckv

struct dckv_plan_s {
  int n_layers, n_kv_heads, head_dim, D, C, hidden, emb, vocab, keep_head, keep_tail;
  float rope_theta, step_scale;
  int C_a, G;
  uint32_t crc;
  int device;
  std::vector<float> step;
  std::vector<uint8_t> active;
  std::vector<uint16_t> freq;  // [C_a][255]
  const uint16_t *A, *S, *W1, *W2, *E, *H;
  dckv::PlanDev dev;
  void *dev_block = nullptr;  // one allocation holding every PlanDev array
  // embedding-mean table [vocab][C] fp32: column i of row v is
  // sum_k E[v][k] H[perm[i]][k].  Plans over the same device, E, H, vocab and
  // column order share one reference-counted copy; mt_perm is that order.
  float *mtab = nullptr;
  std::vector<int32_t> mt_perm;
  uint64_t dev_bytes = 0;  // the plan's own device block
};

namespace dckv {

// ---- request geometry and workspace layout --------------------------------
struct Geometry {
  int64_t T, N, n_kept;
  int64_t n_blk, G, n_groups;
  int64_t N256;       // N rounded up to 256
  int64_t NM;         // N rounded up to kBM
  int64_t n_mtiles;   // NM / kBM
  int64_t Ca4;        // C_a rounded up to kBN
  int64_t esc_cap;    // escape records the encode workspace holds
  int64_t rope_hi;    // ceil(T / 256)
  uint64_t fixed_bytes;  // header + kept rows + group offsets
};

// control block at the start of every workspace (device)
struct Ctrl {
  uint32_t n_esc;        // escapes found (encode) / read (decode)
  int32_t status;        // sticky first error
  uint64_t total_bytes;  // stream size (encode)
  uint64_t rans_bytes;
  uint64_t esc_off;      // byte offset of the escape section in the stream
  uint64_t rans_off;     // byte offset of the rANS section in the stream
  uint64_t offs_off;     // byte offset of the group offsets in the stream
  uint32_t pad[52];
};
static_assert(sizeof(Ctrl) == 256, "ctrl block is 256 bytes");

struct Layout {
  uint64_t ctrl, sym, esc_raw, esc_sorted, halo_a, halo_b, scratch, gwords, goffs;
  uint64_t yhat_b, h_b, w1_part, rope_lo, rope_hi, esc_rows, dhalo, total;
  uint64_t enc_total;  // end of what the encode kernels touch (total covers decode too)
};

Geometry geometry(const dckv_plan_t *p, int64_t T);
Layout layout(const dckv_plan_t *p, const Geometry &g);

// ---- error reporting --------------------------------------------------------
int set_error(int code, const std::string &msg);
int check_hip(hipError_t e, const char *what);

// ---- kernel timing ----------------------------------------------------------
struct KernelTimer {
  KernelTimer(const char *name, hipStream_t s);
  ~KernelTimer();
  const char *name_;
  hipStream_t s_;
  hipEvent_t a_ = nullptr, b_ = nullptr;
};

// ---- launchers (rans.hip / gemm.hip / misc.hip) -----------------------------
struct EncodeArgs {
  const dckv_plan_t *p;
  Geometry g;
  Layout l;
  uint8_t *ws;
  const uint16_t *rows;
  const int32_t *tok;
  uint8_t *stream;
  uint64_t capacity;
  uint64_t *stream_bytes;
  int32_t *status;
  hipStream_t s;
  // set (encode from a post-RoPE cache): the pre-RoPE key heads of every row,
  // [T][kKeyCols]; rows then supplies only the value heads
  const uint16_t *keys = nullptr;
  // set: the call's status starts as *pre (a check run before the encode)
  // instead of 0
  const int32_t *pre = nullptr;
};

// Decoded rows either as rows_out [T][D], or per attention layer: for layer
// l and kv (0 keys, 1 values), heads[2 l + kv] -> [n_kv_heads][T][head_dim]
// (head h of the row's column block (2 l + kv) 2 + h).
struct KvHeads {
  uint16_t *p[12];
};

struct DecodeArgs {
  const dckv_plan_t *p;
  Geometry g;
  Layout l;
  uint8_t *ws;
  const uint8_t *stream;
  uint64_t stream_size;
  const int32_t *tok;
  uint16_t *rows_out;
  int32_t *status;
  hipStream_t s;
  const KvHeads *heads = nullptr;  // set: the per-layer layout, rows_out unused
};

// The stream stages (kept rows, rANS, scan, pack, parse) take n requests at
// once: their kernels run up to kLaunchBatch requests per launch, so the
// requests of a batch share each launch (and its load balance).
constexpr int kLaunchBatch = 16;

// Parameters of up to kMax requests for one launch of a stage kernel:
// request r owns workgroups [start[r], start[r + 1]) of a 1-D grid.
template <class P, int kMax = kLaunchBatch>
struct Batch {
  int n;
  uint32_t start[kMax + 1];
  P r[kMax];
};

// The request that owns workgroup w (a wave-uniform scan of the starts).
template <class P, int kMax>
__device__ __forceinline__ int batch_req(const Batch<P, kMax> &B, uint32_t w) {
  int r = 0;
#pragma unroll
  for (int i = 1; i < kMax; ++i) r = (i < B.n && w >= B.start[i]) ? i : r;
  return r;
}

// Launches kern over requests 0..n-1 in launches of up to kMax: fill(i) gives
// request i's parameters, count(i) its workgroups (0: none); lds, dynamic LDS
// bytes per workgroup.
template <class P, int kMax = kLaunchBatch, class Kern, class Fill, class Count>
void launch_batched(Kern kern, const char *name, int n, hipStream_t s, unsigned threads, Fill fill, Count count,
                    size_t lds = 0) {
  if (lds > 65536)
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds);
  for (int i0 = 0; i0 < n; i0 += kMax) {
    Batch<P, kMax> B{};
    B.n = n - i0 < kMax ? n - i0 : kMax;
    uint32_t w = 0;
    for (int r = 0; r < B.n; ++r) {
      B.start[r] = w;
      B.r[r] = fill(i0 + r);
      w += count(i0 + r);
    }
    for (int r = B.n; r <= kMax; ++r) B.start[r] = w;
    if (w == 0) continue;
    KernelTimer tm(name, s);
    hipLaunchKernelGGL(kern, dim3(w), dim3(threads), lds, s, B);
  }
}

// A paged attention cache: per layer l, a key (kv = 0) and a value (kv = 1)
// pool p[2 l + kv] of [n_blocks][block_size][n_kv_heads][head_dim] bf16;
// position t of a request is row table[t / bs] * bs + t % bs of every pool.
struct PagedKV {
  uint16_t *p[12];
  const int32_t *table;
  int32_t bs;
  int64_t n_blocks;
};

// misc.hip
void launch_start_encode(const EncodeArgs *a, int n);  // control words, status, kept rows
// status := EINVAL when an entry of the first ceil(T / bs) of the block table
// is outside [0, n_blocks); clear_first: set it to 0 before (else only set)
void launch_paged_check(const PagedKV &kv, int64_t T, int32_t *status, bool clear_first, hipStream_t s);
// rows [T][D] <- the paged cache (post_rope: keys rotated back, as dckv_unrope);
// nothing is read when *pre is not 0
void launch_paged_gather(const dckv_plan_t *p, const PagedKV &kv, bool post_rope, int64_t T, uint16_t *rows,
                         const int32_t *pre, hipStream_t s);
// the paged cache <- rows [T][D]; nothing is written when *status is not 0
void launch_paged_scatter(const PagedKV &kv, int64_t T, const uint16_t *rows, const int32_t *status, hipStream_t s);
void launch_unrope(const dckv_plan_t *p, const uint16_t *in, uint16_t *out, int64_t T, hipStream_t s);
// the inverse RoPE of the key heads only, rows [T][D] -> keys [T][kKeyCols]
void launch_unrope_keys(const dckv_plan_t *p, const uint16_t *in, uint16_t *keys, int64_t T, hipStream_t s);

// The rANS decoder also dequantises (writes yhat_b) for a request whose plan
// codes every component (a full decode: token ids given); k_dequant then
// skips it.
inline bool dequant_fused(const DecodeArgs &a) {
  return a.g.N > 0 && a.tok != nullptr && a.p->C_a == a.p->C && a.p->C == kC;
}

// rans.hip
void launch_rans_encode(const EncodeArgs *a, int n);
void launch_scan_header(const EncodeArgs *a, int n);
void launch_pack(const EncodeArgs *a, int n);
void launch_parse(const DecodeArgs *a, int n, bool with_rope);  // control words, status, parse, RoPE tables
void launch_rans_decode(const DecodeArgs *a, int n);
void launch_load_esc(const EncodeArgs &a, const uint32_t *esc, uint32_t n_esc);
void launch_sym_to_tiled(const EncodeArgs &a, const uint8_t *sym);
void launch_sym_from_tiled(const DecodeArgs &a, uint8_t *sym_out, uint32_t *n_esc_out);

// gemm.hip
int build_mean_table(dckv_plan_t *p);  // at plan time: fills p->mtab, synchronous

// C[m][n] = sum_k A[m][k] B[n][k], bf16 operands (k contiguous), fp32 output.
// k-tiles [0, split) read a0 / b0, the rest a1 / b1 (row bytes lda*, ldb*);
// A's row m is arow[m] when arow is set.  K = 64 KT; N a multiple of 8 tiles
// of 256 or at most 8 of them (the tile order's grouping).
struct GemmF32Args {
  const uint16_t *a0, *a1, *b0, *b1;
  uint32_t lda0, lda1, ldb0, ldb1;
  int split, KT;
  const int32_t *arow;
  int M, N;
  float *c;
  int64_t ldc;
  // ksplit > 1 (single-source operands, KT a multiple of ksplit): slice ks of
  // the k range goes to c + ks * M * ldc, for the caller to add up
  int ksplit;
  int n_mt, n_nt;  // set by the launcher
};
void launch_gemm_f32(const GemmF32Args &args, hipStream_t s);
// two independent products in one launch (the second's workgroups follow the first's)
void launch_gemm_f32_pair(const GemmF32Args &a, const GemmF32Args &b, hipStream_t s);

// fit.hip: the closed-form fit of the conditional models
constexpr int kFitChunks = 512;  // row chunks of the per-component sums
struct FitLayout {
  int64_t n_pad = 0;  // n rounded up to 64 (the inner dimension of the Gram products)
  uint64_t Y = 0, M = 0, Yhi = 0, Ylo = 0, Et = 0, G = 0, R = 0, Hb = 0, tokc = 0, part = 0, dg = 0, linv = 0, total = 0;
};
FitLayout fit_layout(int64_t n);
struct FitArgs {
  FitLayout l;
  uint8_t *ws;
  const uint16_t *rows, *A, *E;
  const int32_t *tok;
  int64_t n;
  int vocab;
  float ridge;
  float *H_out;       // may be null
  uint16_t *Hb_out;   // may be null
  float *a_out, *b_out;
  int32_t *status;
  hipStream_t s;
};
void fit_sequence(const FitArgs &a);
// shared with the rate's weight gradients: clear a status word; gather E[tok]
// transposed to [emb][n_pad] bf16 (EINVAL for a bad id); split fp32 [n][C]
// into transposed bf16 high and low halves [C][n_pad] (zero past n)
void launch_clear_status(int32_t *status, hipStream_t s);
void launch_gather_t(const uint16_t *E, const int32_t *tok, int64_t n, int64_t n_pad, int vocab, uint16_t *Et,
                     int32_t *tokc, int32_t *status, hipStream_t s);
void launch_split_t(const float *Y, int64_t n, int64_t n_pad, uint16_t *hi, uint16_t *lo, hipStream_t s);

// rate.hip: the training rate (additive-noise likelihood) and its gradients
struct RateLayout {
  int64_t chunks = 0;  // row chunks of the rate kernel
  int64_t parts = 0;   // partial rows of the per-component sums (one per chunk)
  int ksplit = 1;      // k-slices of the transform (partial coefficient sets)
  int64_t n_seg = 0;   // first-stage segments of those sums
  uint64_t Y = 0, bits_part = 0, ga_part = 0, gb_part = 0, flags = 0, ga_seg = 0, gb_seg = 0, flags2 = 0, total = 0;
};
RateLayout rate_layout(int64_t N);
struct RateArgs {
  const dckv_plan_t *p;
  RateLayout l;
  uint8_t *ws;
  const uint16_t *rows;
  const int32_t *tok;
  const float *noise;
  int64_t N;
  float *bits, *yhat, *grad_y, *grad_mean, *grad_nbr, *grad_scale;
  int32_t *status;
  hipStream_t s;
};
void rate_sequence(const RateArgs &a);
// the weight gradients dR/dA = G_y^T X and dR/dH = G_m^T E[tok]
struct RateBwdLayout {
  int64_t n_pad = 0;  // N rounded up to 64 (the inner dimension)
  uint64_t gy_hi = 0, gy_lo = 0, gm_hi = 0, gm_lo = 0, Xt = 0, Et = 0, tokc = 0, total = 0;
};
RateBwdLayout rate_bwd_layout(int64_t N);
struct RateBwdArgs {
  const dckv_plan_t *p;
  RateBwdLayout l;
  uint8_t *ws;
  const uint16_t *rows;
  const int32_t *tok;
  const float *grad_y, *grad_mean;
  int64_t N;
  float *grad_A, *grad_H;
  int32_t *status;
  hipStream_t s;
};
void rate_bwd_sequence(const RateBwdArgs &a);
void launch_analysis_gemm(const EncodeArgs *a, int n);
void launch_encode_fixup(const EncodeArgs *a, int n);
void launch_dequant(const DecodeArgs *a, int n);
void launch_w1_gemm(const DecodeArgs *a, int n);
void launch_synthesis_gemm(const DecodeArgs *a, int n);


}  // namespace dckv
