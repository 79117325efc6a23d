// Lossless stage of the DCKV codec on gfx950: interleaved 32-bit rANS over
// (256-token block, 64 active components) groups, the stream writer and the
// stream parser.
//
// Source: DCKV digest page ("DCKV: Learned Transform Coding of the Prompt KV
// Cache in Hybrid Language Models"), "How it works", Coding bullet: codes are
// rANS-coded on the GPU under Laplace distributions and codes beyond +-127
// are escaped at 64 bits each.  Coder parameters and layout are this
// library's own (stream version 1): 32-bit state, L = 2^16, 16-bit words,
// 15-bit tables, one group = one wave64 whose lanes are the group's
// components.
//
// Encoder: every lane starts at L; tokens go last to first; a lane whose
// state is >= f * 2^17 emits its low 16 bits before coding.  All lanes of a
// step emit at once; the step's words are ordered by descending lane (a
// ballot plus a popcount of the higher lanes gives each lane its slot), so
// that after the final reversal the decoder reads them by ascending lane.
// Decoder: the same machine run forwards, one step per token for all 64
// lanes, words taken by ascending lane (ballot plus a popcount of the lower
// lanes).  A group is valid only if every lane ends at L and every word was
// consumed.
#include "dckv_internal.h"

namespace dckv {
namespace {

constexpr int kTabStride = 257;   // u32 per table row in LDS: spreads equal symbols over banks
constexpr int kEncWaves = 16;     // groups (waves) per encoder workgroup, one component group
constexpr int kDecWaves = 16;
constexpr int kWordBuf = 1024;    // u16 words cached per decoder wave
constexpr int kBktStride = kBuckets + 4;  // bytes per bucket row in LDS (65 dwords: rows on distinct banks)

__device__ __forceinline__ void set_status(int32_t *st, int code) { atomicCAS(st, 0, code); }

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// A load through a global (address space 1) pointer.
template <class T>
__device__ __forceinline__ T gload(const T *p) {
  return *(const T __attribute__((address_space(1))) *)p;
}

// The tables of component group g into LDS: n rows of 256 u32 (LDS row stride
// kTabStride), contiguous in the plan.  Every thread issues its 16-byte loads
// before its first LDS write, so the copy costs one memory latency.
template <int kThreads>
__device__ __forceinline__ void stage_tab(uint32_t *tab, const uint32_t *gtab, int g, int n) {
  constexpr int kPer = kLanes * 256 / 4 / kThreads;  // 16-byte pieces per thread
  static_assert(kPer * kThreads * 4 == kLanes * 256, "whole pieces");
  const u32x4 *src = reinterpret_cast<const u32x4 *>(gtab + (size_t)kLanes * g * 256);
  u32x4 v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int pc = threadIdx.x + i * kThreads;  // row pc / 64, entries 4 (pc % 64) ..
    if ((pc >> 6) < n) v[i] = gload(src + pc);
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int pc = threadIdx.x + i * kThreads;
    if ((pc >> 6) < n) {
      uint32_t *d = tab + (pc >> 6) * kTabStride + (pc & 63) * 4;
      d[0] = v[i].x;
      d[1] = v[i].y;
      d[2] = v[i].z;
      d[3] = v[i].w;
    }
  }
}

__device__ __forceinline__ Ctrl *ctrl_of(uint8_t *ws) { return reinterpret_cast<Ctrl *>(ws); }

struct EncP {
  const uint32_t *tab;     // [C_a][256]
  const uint32_t *sym32;   // tiled symbols
  uint16_t *scratch;       // [n_groups][64 * 258]
  uint32_t *gwords;        // [n_groups]
  int64_t N, N256, n_blk;
  int Ca, G;
  const int32_t *status;
};

__global__ __launch_bounds__(kEncWaves * 64) void k_rans_encode(EncP P) {
  __shared__ uint32_t tab[kLanes * kTabStride];
  const int g = blockIdx.y;
  const int n = min(kLanes, P.Ca - kLanes * g);
  stage_tab<kEncWaves * 64>(tab, P.tab, g, n);
  __syncthreads();
  if (*P.status != 0) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t b = (int64_t)blockIdx.x * kEncWaves + wave;
  if (b >= P.n_blk) return;
  const int Lb = (int)min<int64_t>(kBlock, P.N - kBlock * b);
  const int64_t gid = b * P.G + g;
  const uint32_t *sw = P.sym32 + ((size_t)g * (P.N256 / 4) + (size_t)b * 64) * 64 + lane;
  uint16_t *out = P.scratch + (size_t)gid * (kLanes * (kBlock + 2));
  const bool lane_ok = lane < n;
  // Escapes code as the identity: table entry 255 is f = 2^15, cum = 0, so
  // the state never emits and x / f * 2^15 + x % f = x.  Lanes past C_a code
  // escapes only, through lane 0's table row.
  const uint32_t *mytab = tab + (lane_ok ? lane : 0) * kTabStride;
  uint32_t x = kL;
  uint32_t cnt = 0;
  auto enc = [&](uint32_t s) {
    const uint32_t e = mytab[s];
    const uint32_t f = e & 0xFFFFu, c = e >> 16;
    const bool emit = (x >> 17) >= f;  // x >= f 2^17 (f = 2^15 never emits)
    const uint64_t mask = __ballot(emit);
    if (mask) {
      // the emitting lanes write in descending lane order
      const uint32_t tot = (uint32_t)__popcll(mask);
      const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
      if (emit) out[cnt + tot - 1u - below] = (uint16_t)(x & 0xFFFFu);
      x = emit ? x >> 16 : x;
      cnt += tot;
    }
    // x / f within one from a float reciprocal (x < f 2^17), then corrected
    const uint32_t q0 = (uint32_t)((float)x * __builtin_amdgcn_rcpf((float)f));
    int32_t r = (int32_t)(x - __umul24(q0, f));
    const uint32_t neg = (uint32_t)r >> 31;
    r += neg ? (int32_t)f : 0;
    const uint32_t big = r >= (int32_t)f;
    r -= big ? (int32_t)f : 0;
    x = ((q0 - neg + big) << kPrecBits) + (uint32_t)r + c;
  };
  // symbol words in chunks of 8 quads, last chunk first; the words of the
  // next chunk are loaded while this one is coded (every quad of the block
  // is in the buffer; quads past the last are not coded)
  const int nq = (Lb + 3) >> 2;
  const int nch = (nq + 7) >> 3;
  // rows past the block in its last quad code as escapes
  const uint32_t tail = (Lb & 3) ? 0xFFFFFFFFu << (8 * (Lb & 3)) : 0u;
  uint32_t wq[8], wn[8];
  auto load_chunk = [&](int ch, uint32_t (&w)[8]) {
#pragma unroll
    for (int u = 0; u < 8; ++u) w[u] = gload(sw + (size_t)(ch * 8 + u) * 64);
  };
  load_chunk(nch - 1, wn);
#pragma unroll 1
  for (int ch = nch - 1; ch >= 0; --ch) {
#pragma unroll
    for (int u = 0; u < 8; ++u) wq[u] = lane_ok ? wn[u] : 0xFFFFFFFFu;
    if (ch > 0) load_chunk(ch - 1, wn);
#pragma unroll
    for (int u = 7; u >= 0; --u) {
      const int qd = ch * 8 + u;
      if (qd >= nq) continue;
      const uint32_t w = wq[u] | (qd == nq - 1 ? tail : 0u);
#pragma unroll
      for (int k = 3; k >= 0; --k) enc((w >> (8 * k)) & 0xFFu);
    }
  }
  if (lane_ok) {
    const uint32_t pos = cnt + 2u * (uint32_t)(n - 1 - lane);
    out[pos] = (uint16_t)(x >> 16);
    out[pos + 1] = (uint16_t)(x & 0xFFFFu);
  }
  if (lane == 0) P.gwords[gid] = cnt + 2u * (uint32_t)n;
}

// ---------------------------------------------------------------------------
// group-size scan, group offsets, header, final size
// ---------------------------------------------------------------------------
// Escapes (codes beyond +-127, 64 bits each) are found out of order by the
// quantiser tiles; the stream stores them by ascending flat index
// j * C_a + rank, so the scan's workgroup first sorts the (usually few)
// records with a bitonic network, in LDS up to kSortLds records, else in
// place in global memory.
constexpr int kSortLds = 4096;

__device__ __forceinline__ void bitonic(unsigned long long *a, uint32_t n_pow2) {
  for (uint32_t k = 2; k <= n_pow2; k <<= 1) {
    for (uint32_t j = k >> 1; j > 0; j >>= 1) {
      for (uint32_t i = threadIdx.x; i < n_pow2; i += blockDim.x) {
        const uint32_t l = i ^ j;
        if (l > i) {
          const unsigned long long x = a[i], y = a[l];
          const bool up = (i & k) == 0;
          if ((x > y) == up) {
            a[i] = y;
            a[l] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

// esc_raw holds {flat, q} pairs in arrival order; esc_sorted receives them by
// ascending flat.  esc_raw has room for the padded power-of-two count.  All
// threads of the workgroup call this.
__device__ __forceinline__ void sort_escapes(const uint8_t *ws, uint32_t *esc_raw, uint32_t *esc_sorted,
                                             int64_t esc_cap, unsigned long long *keys) {
  const Ctrl *ct = reinterpret_cast<const Ctrl *>(ws);
  const uint32_t n = (uint32_t)min<int64_t>(ct->n_esc, esc_cap);
  if (n == 0) return;
  uint32_t p2 = 1;
  while (p2 < n) p2 <<= 1;
  unsigned long long *a;
  unsigned long long *g = reinterpret_cast<unsigned long long *>(esc_raw);
  if (p2 <= (uint32_t)kSortLds) {
    a = keys;
    for (uint32_t i = threadIdx.x; i < p2; i += blockDim.x)
      a[i] = i < n ? (((unsigned long long)esc_raw[2 * i]) << 32) | esc_raw[2 * i + 1] : ~0ull;
  } else {
    // in place in global memory: keys overwrite the pairs they were made from
    a = g;
    for (uint32_t i = threadIdx.x; i < p2; i += blockDim.x) {
      unsigned long long v = ~0ull;
      if (i < n) v = (((unsigned long long)esc_raw[2 * i]) << 32) | esc_raw[2 * i + 1];
      a[i] = v;  // element i occupies exactly the bytes of pair i
    }
  }
  __syncthreads();
  bitonic(a, p2);
  for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) {
    const unsigned long long v = a[i];
    esc_sorted[2 * i] = (uint32_t)(v >> 32);
    esc_sorted[2 * i + 1] = (uint32_t)v;
  }
}

struct ScanP {
  uint32_t *esc_raw, *esc_sorted;
  const uint32_t *gwords;
  uint64_t *goffs;        // word offsets [n_groups + 1]
  uint8_t *ws;
  uint8_t *stream;
  uint64_t capacity;
  uint64_t *stream_bytes;
  int32_t *status;
  int64_t n_groups, esc_cap;
  uint64_t kept_bytes;
  uint32_t T, keep_head, keep_tail, N, n_coef, Ca, crc;
  float step_scale;
};

__global__ __launch_bounds__(1024) void k_scan_header(ScanP P) {
  __shared__ uint64_t part[1024];
  __shared__ unsigned long long keys[kSortLds];
  const int t = threadIdx.x;
  if (*P.status == 0) sort_escapes(P.ws, P.esc_raw, P.esc_sorted, P.esc_cap, keys);
  __syncthreads();
  const int64_t ng = P.n_groups;
  const int64_t per = (ng + 1023) / 1024;
  const int64_t lo = min<int64_t>(ng, t * per), hi = min<int64_t>(ng, lo + per);
  uint64_t s = 0;
  for (int64_t i = lo; i < hi; ++i) s += P.gwords[i];
  // inclusive scan: within each wave by shuffles, then the 16 wave totals
  const int lane = t & 63, wv = t >> 6;
  uint64_t incl = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) part[wv] = incl;
  __syncthreads();
  uint64_t before = 0;
  for (int w = 0; w < wv; ++w) before += part[w];
  uint64_t all = 0;
  for (int w = 0; w < 16; ++w) all += part[w];
  uint64_t run = before + incl - s;
  for (int64_t i = lo; i < hi; ++i) {
    P.goffs[i] = run;
    run += P.gwords[i];
  }
  const uint64_t total_words = all;
  if (t == 0) P.goffs[ng] = total_words;
  Ctrl *ct = ctrl_of(P.ws);
  const uint32_t n_esc = ct->n_esc;
  const uint64_t offs_off = kHeaderBytes + P.kept_bytes;
  const uint64_t esc_off = offs_off + 4ull * (ng + 1);
  const uint64_t rans_off = esc_off + 8ull * n_esc;
  const uint64_t total = rans_off + 2ull * total_words;
  __syncthreads();
  int32_t st = *P.status;
  if (st == 0 && n_esc > (uint64_t)P.esc_cap) st = DCKV_ECAPACITY;
  if (st == 0 && total > P.capacity) st = DCKV_ECAPACITY;
  if (t == 0) {
    ct->total_bytes = st == 0 ? total : 0;
    ct->rans_bytes = 2ull * total_words;
    ct->esc_off = esc_off;
    ct->rans_off = rans_off;
    ct->offs_off = offs_off;
    if (st != 0) set_status(P.status, st);
    *P.stream_bytes = st == 0 ? total : 0;
  }
  if (st != 0) return;
  uint32_t *offs32 = reinterpret_cast<uint32_t *>(P.stream + offs_off);
  for (int64_t i = t; i <= ng; i += 1024) offs32[i] = (uint32_t)(2ull * (i == ng ? total_words : P.goffs[i]));
  if (t < 16) {
    uint32_t v = 0;
    switch (t) {
      case 0: v = 0x564B4344u; break;                       // "DCKV"
      case 1: v = (uint32_t)kVersion | ((uint32_t)kHeaderBytes << 16); break;
      case 2: v = P.T; break;
      case 3: v = P.keep_head; break;
      case 4: v = P.keep_tail; break;
      case 5: v = P.N; break;
      case 6: v = P.n_coef; break;
      case 7: v = P.Ca; break;
      case 8: v = (uint32_t)ng; break;
      case 9: v = n_esc; break;
      case 10: v = __float_as_uint(P.step_scale); break;
      case 11: v = P.crc; break;
      case 12: v = (uint32_t)total; break;
      case 13: v = (uint32_t)(total >> 32); break;
      case 14: v = (uint32_t)(2ull * total_words); break;
      case 15: v = (uint32_t)((2ull * total_words) >> 32); break;
    }
    reinterpret_cast<uint32_t *>(P.stream)[t] = v;
  }
}

// ---------------------------------------------------------------------------
// pack: reversed group words and the escape records into the stream
// ---------------------------------------------------------------------------
struct PackP {
  const uint16_t *scratch;
  const uint32_t *gwords;
  const uint64_t *goffs;
  const uint32_t *esc_sorted;  // {flat, q} pairs
  uint8_t *ws;
  uint8_t *stream;
  int64_t n_groups;
  const int32_t *status;
};

__global__ __launch_bounds__(256) void k_pack(PackP P) {
  if (*P.status != 0) return;
  const Ctrl *ct = reinterpret_cast<const Ctrl *>(P.ws);
  const uint64_t rans_off = ct->rans_off, esc_off = ct->esc_off;
  const uint32_t n_esc = ct->n_esc;
  for (int64_t gid = blockIdx.x; gid < P.n_groups; gid += gridDim.x) {
    const uint32_t W = P.gwords[gid];
    const uint16_t *src = P.scratch + (size_t)gid * (kLanes * (kBlock + 2));
    uint16_t *dst = reinterpret_cast<uint16_t *>(P.stream + rans_off) + P.goffs[gid];
    for (uint32_t k = threadIdx.x; k < W; k += blockDim.x) dst[k] = src[W - 1 - k];
  }
  uint32_t *e = reinterpret_cast<uint32_t *>(P.stream + esc_off);
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n_esc; i += gridDim.x * blockDim.x) {
    e[2 * i] = P.esc_sorted[2 * i];
    e[2 * i + 1] = P.esc_sorted[2 * i + 1];
  }
}

// ---------------------------------------------------------------------------
// parse: validate a stream against the plan and the request
// ---------------------------------------------------------------------------
struct ParseP {
  const uint8_t *stream;
  uint64_t size;
  uint8_t *ws;
  int32_t *status;
  // RoPE angle tables, built by the workgroups after the first (none when
  // n_rope is 0): lo[u][i] = (cos, sin)(u w_i), u < 256; hi[v][i] = the same
  // of 256 v w_i; in float64, rounded once
  const double *omega;
  float2 *rope_lo, *rope_hi;
  int64_t rope_hi_n;
  uint32_t T, keep_head, keep_tail, N, n_coef, Ca, crc, n_groups;
  uint64_t kept_bytes;
  uint32_t *esc_rows;     // [row tiles][2]: index range of the escapes of a 256-row tile
  uint32_t n_row_tiles;
};

__global__ __launch_bounds__(256) void k_parse(ParseP P) {
  __shared__ int bad;
  __shared__ int plan_bad;
  __shared__ uint64_t s_esc_off, s_rans_off, s_rans_bytes;
  __shared__ uint32_t s_n_esc;
  const int t = threadIdx.x;
  if (blockIdx.x > 0) {
    const int64_t n = (256 + P.rope_hi_n) * kHalf;
    for (int64_t i = (int64_t)(blockIdx.x - 1) * blockDim.x + t; i < n; i += (int64_t)(gridDim.x - 1) * blockDim.x) {
      const int64_t u = i / kHalf;
      const int k = (int)(i - u * kHalf);
      double ang;
      float2 *dst;
      if (u < 256) {
        ang = (double)u * P.omega[k];
        dst = P.rope_lo + u * kHalf + k;
      } else {
        ang = (double)((u - 256) * 256) * P.omega[k];
        dst = P.rope_hi + (u - 256) * kHalf + k;
      }
      double sn, cs;
      sincos(ang, &sn, &cs);
      *dst = make_float2((float)cs, (float)sn);
    }
    return;
  }
  if (t == 0) {  // the call's control words and status start clear
    Ctrl *ct = ctrl_of(P.ws);
    ct->n_esc = 0;
    ct->status = 0;
    ct->total_bytes = 0;
    ct->rans_bytes = 0;
    ct->esc_off = ct->rans_off = ct->offs_off = 0;
    *P.status = 0;
  }
  __syncthreads();
  for (uint32_t i = t; i < 2 * P.n_row_tiles; i += blockDim.x) P.esc_rows[i] = 0u;  // no records
  if (t == 0) {
    bad = 0;
    plan_bad = 0;
    const uint32_t *h = reinterpret_cast<const uint32_t *>(P.stream);
    if (P.size < (uint64_t)kHeaderBytes || h[0] != 0x564B4344u ||
        h[1] != ((uint32_t)kVersion | ((uint32_t)kHeaderBytes << 16))) {
      bad = 1;
    } else {
      if (h[11] != P.crc || h[7] != P.Ca || h[6] != P.n_coef) plan_bad = 1;
      if (h[2] != P.T || h[3] != P.keep_head || h[4] != P.keep_tail || h[5] != P.N || h[8] != P.n_groups)
        bad = 1;
      const uint32_t n_esc = h[9];
      const uint64_t total = (uint64_t)h[12] | ((uint64_t)h[13] << 32);
      const uint64_t rb = (uint64_t)h[14] | ((uint64_t)h[15] << 32);
      const uint64_t offs_off = kHeaderBytes + P.kept_bytes;
      const uint64_t esc_off = offs_off + 4ull * ((uint64_t)P.n_groups + 1);
      if ((uint64_t)n_esc > (uint64_t)P.N * P.Ca) bad = 1;
      const uint64_t rans_off = esc_off + 8ull * n_esc;
      if (rb > P.size || total > P.size || rans_off + rb != total || (rb & 1)) bad = 1;
      s_n_esc = n_esc;
      s_esc_off = esc_off;
      s_rans_off = rans_off;
      s_rans_bytes = rb;
    }
  }
  __syncthreads();
  if (!bad && !plan_bad) {
    const uint32_t *offs = reinterpret_cast<const uint32_t *>(P.stream + kHeaderBytes + P.kept_bytes);
    int my_bad = 0;
    for (uint32_t i = t; i < P.n_groups; i += blockDim.x) {
      const uint32_t a = offs[i], b2 = offs[i + 1];
      if (b2 < a || (a & 1) || (b2 & 1)) my_bad = 1;
    }
    if (t == 0 && (offs[0] != 0 || (uint64_t)offs[P.n_groups] != s_rans_bytes)) my_bad = 1;
    const uint32_t *esc = reinterpret_cast<const uint32_t *>(P.stream + s_esc_off);
    const uint64_t lim = (uint64_t)P.N * P.Ca;
    for (uint32_t i = t; i < s_n_esc; i += blockDim.x) {
      const uint32_t f = esc[2 * i];
      if ((uint64_t)f >= lim) {
        my_bad = 1;
      } else {
        // the first / one-past-last escape of its 256-row tile
        const uint32_t mt = (f / P.Ca) >> 8;
        if (i == 0 || (esc[2 * i - 2] / P.Ca) >> 8 != mt) P.esc_rows[2 * mt] = i;
        if (i + 1 == s_n_esc || (esc[2 * i + 2] / P.Ca) >> 8 != mt) P.esc_rows[2 * mt + 1] = i + 1;
      }
      if (i + 1 < s_n_esc && esc[2 * i + 2] <= f) my_bad = 1;
    }
    if (my_bad) atomicOr(&bad, 1);
  }
  __syncthreads();
  if (t == 0) {
    Ctrl *ct = ctrl_of(P.ws);
    if (plan_bad) set_status(P.status, DCKV_EPLAN);
    else if (bad) set_status(P.status, DCKV_ECORRUPT);
    ct->n_esc = bad || plan_bad ? 0 : s_n_esc;
    ct->esc_off = s_esc_off;
    ct->rans_off = s_rans_off;
    ct->offs_off = kHeaderBytes + P.kept_bytes;
    ct->rans_bytes = s_rans_bytes;
  }
}

// ---------------------------------------------------------------------------
// decoder
// ---------------------------------------------------------------------------
struct DecP {
  const uint32_t *tab;
  const uint8_t *bucket;
  const uint8_t *stream;
  const uint8_t *ws;
  const uint32_t *esc_rows;  // [blocks][2]: index range of each block's escape records (from the parser)
  uint32_t *sym32;
  int64_t N, N256, n_blk;
  int Ca, G;
  int32_t *status;
};

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The symbols of one wave's rows: step i pops the symbol of row i from each
// lane's state (bucket of the slot, then a binary search while any lane's
// bucket holds more than one symbol), then renormalises the lanes that need
// it with the next words of the interleaved stream, in lane order.  kPlain:
// every lane is a coded component and the block has no escapes, so no lane
// is ever skipped.  The word window is read modulo its size: a valid stream
// never leaves it (it slides before it would), and a corrupt one ends with
// ptr != W or a final state != L, which the caller reports.
template <bool kPlain>
__device__ __forceinline__ void decode_rows(uint32_t &x, uint32_t &ptr, uint32_t &base, uint32_t W, int Lb, int lane,
                                            bool lane_ok, const unsigned long long *ebits, const uint32_t *mytab,
                                            const uint8_t *mybkt, uint16_t *wb, const uint16_t *wsrc,
                                            uint32_t *sout) {
  auto step = [&](int i) -> uint32_t {
    bool act = true;
    if (!kPlain) {
      act = lane_ok;
      if (ebits) act = act && !((ebits[i] >> lane) & 1ull);
    }
    const uint32_t slot = x & (kM - 1u);
    const uint32_t bi = slot >> kBucketShift;
    uint32_t lo = mybkt[bi];
    uint32_t hi = mybkt[bi + 1];
    if (!kPlain) hi = act ? hi : lo;
    while (__ballot(lo < hi)) {
      const uint32_t mid = (lo + hi + 1) >> 1;
      const bool up = (mytab[mid] >> 16) <= slot;
      const bool open = lo < hi;
      lo = open && up ? mid : lo;
      hi = open && !up ? mid - 1 : hi;
    }
    const uint32_t e = mytab[lo];
    // f * (x >> 15) < 2^32: f <= 2^15 and x >> 15 < 2^17 (24-bit multiply)
    const uint32_t xd = __umul24(e & 0xFFFFu, x >> kPrecBits) + slot - (e >> 16);
    x = act ? xd : x;
    const bool need = act && x < kL;
    const uint64_t mask = __ballot(need);
    if (mask) {
      const uint32_t cnt = (uint32_t)__popcll(mask);
      if (ptr + cnt > base + kWordBuf && base + kWordBuf < W) {  // slide the window
        base = ptr;
        wave_sync_lds();
        for (uint32_t k = lane; k < kWordBuf && base + k < W; k += 64) wb[k] = wsrc[base + k];
        wave_sync_lds();
      }
      const uint32_t before = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
      const uint32_t wv = wb[(ptr - base + before) & (kWordBuf - 1u)];
      x = need ? (x << 16) | wv : x;
      ptr += cnt;
    }
    return act ? lo : (uint32_t)kEsc;
  };
  const int nq = Lb >> 2;
#pragma unroll 1
  for (int q = 0; q < nq; ++q) {
    uint32_t w = step(4 * q);
    w |= step(4 * q + 1) << 8;
    w |= step(4 * q + 2) << 16;
    w |= step(4 * q + 3) << 24;
    if (kPlain || lane_ok) sout[(size_t)q * 64] = w;
  }
  if (Lb & 3) {  // the last, partial quad: rows past the block read as escapes
    uint32_t w = 0xFFFFFFFFu;
#pragma unroll 1
    for (int k = 0; k < (Lb & 3); ++k) w = (w & ~(0xFFu << (8 * k))) | (step(4 * nq + k) << (8 * k));
    if (kPlain || lane_ok) sout[(size_t)nq * 64] = w;
  }
}

__global__ __launch_bounds__(kDecWaves * 64) void k_rans_decode(DecP P) {
  __shared__ uint32_t tab[kLanes * kTabStride];
  __shared__ uint8_t bkt[kLanes * kBktStride];
  __shared__ uint16_t wbuf[kDecWaves][kWordBuf];
  __shared__ unsigned long long ebits[kDecWaves][kBlock];
  const int g = blockIdx.y;
  const int n = min(kLanes, P.Ca - kLanes * g);
  stage_tab<kDecWaves * 64>(tab, P.tab, g, n);
  {
    // bucket row of lane l: first symbol of each slot bucket, then the last
    // symbol as the upper bound of the last bucket; one 16-byte piece per
    // thread
    static_assert(kDecWaves * 64 * 16 == kLanes * kBuckets, "one piece per thread");
    const int pc = threadIdx.x, l = pc >> 4;
    if (l < n) {
      const u32x4 v = gload(reinterpret_cast<const u32x4 *>(P.bucket + (size_t)kLanes * g * kBuckets) + pc);
      uint32_t *d = reinterpret_cast<uint32_t *>(bkt + l * kBktStride + (pc & 15) * 16);
      d[0] = v.x;
      d[1] = v.y;
      d[2] = v.z;
      d[3] = v.w;
    }
    if (pc < n) bkt[pc * kBktStride + kBuckets] = (uint8_t)(kNSym - 1);
  }
  __syncthreads();
  if (*P.status != 0) return;
  // per-wave values are kept in scalar registers: the step loop is uniform,
  // and lanes that decode nothing at a step take the same path with their
  // results discarded
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t b = (int64_t)blockIdx.x * kDecWaves + wave;
  if (b >= P.n_blk) return;
  const Ctrl *ct = reinterpret_cast<const Ctrl *>(P.ws);
  const int Lb = (int)min<int64_t>(kBlock, P.N - kBlock * b);
  const int64_t gid = b * P.G + g;
  const uint32_t *offs = reinterpret_cast<const uint32_t *>(P.stream + ct->offs_off);
  const uint32_t o0 = offs[gid], o1 = offs[gid + 1];
  const uint16_t *wsrc = reinterpret_cast<const uint16_t *>(P.stream + ct->rans_off + o0);
  const uint32_t W = (o1 - o0) >> 1;
  uint16_t *wb = wbuf[wave];
  const bool lane_ok = lane < n;
  if (W < 2u * (uint32_t)n) {
    if (lane == 0) set_status(P.status, DCKV_ECORRUPT);
    return;
  }
  // escape positions of this group
  const uint32_t *esc = reinterpret_cast<const uint32_t *>(P.stream + ct->esc_off);
  bool has_esc = false;
  {
    // the block's records, as the parser found them (a block is 256 rows)
    const uint32_t lo = __builtin_amdgcn_readfirstlane(gload(P.esc_rows + 2 * b));
    const uint32_t lo2 = __builtin_amdgcn_readfirstlane(gload(P.esc_rows + 2 * b + 1));
    if (lo2 > lo) {
      has_esc = true;
      for (int i = lane; i < kBlock; i += 64) ebits[wave][i] = 0ull;
      wave_sync_lds();
      for (uint32_t e = lo + lane; e < lo2; e += 64) {
        const uint64_t f = esc[2 * e];
        const uint64_t jj = f / (uint64_t)P.Ca;
        const int r = (int)(f - jj * (uint64_t)P.Ca);
        if (r >= kLanes * g && r < kLanes * g + n)
          atomicOr(&ebits[wave][(int)(jj - (uint64_t)kBlock * b)], 1ull << (r - kLanes * g));
      }
      wave_sync_lds();
    }
  }
  // word window [base, base + kWordBuf); the first window's loads are all
  // issued before the first LDS write
  uint32_t base = 0;
  {
    uint16_t v[kWordBuf / 64];
#pragma unroll
    for (int i = 0; i < kWordBuf / 64; ++i) {
      const uint32_t k = (uint32_t)lane + 64u * i;
      if (k < W) v[i] = gload(wsrc + k);
    }
#pragma unroll
    for (int i = 0; i < kWordBuf / 64; ++i) {
      const uint32_t k = (uint32_t)lane + 64u * i;
      if (k < W) wb[k] = v[i];
    }
  }
  wave_sync_lds();
  uint32_t x = kL;
  if (lane_ok) x = (uint32_t)wb[2 * lane] | ((uint32_t)wb[2 * lane + 1] << 16);
  uint32_t ptr = 2u * (uint32_t)n;
  const uint32_t *mytab = tab + lane * kTabStride;
  const uint8_t *mybkt = bkt + lane * kBktStride;
  uint32_t *sout = P.sym32 + ((size_t)g * (P.N256 / 4) + (size_t)b * 64) * 64 + lane;
  const unsigned long long *eb = ebits[wave];
  if (!has_esc && n == kLanes)
    decode_rows<true>(x, ptr, base, W, Lb, lane, true, eb, mytab, mybkt, wb, wsrc, sout);
  else
    decode_rows<false>(x, ptr, base, W, Lb, lane, lane_ok, has_esc ? eb : nullptr, mytab, mybkt, wb, wsrc, sout);
  const bool lane_bad = lane_ok && x != kL;
  if (__ballot(lane_bad) != 0ull || ptr != W) {
    if (lane == 0) set_status(P.status, DCKV_ECORRUPT);
  }
}

// ---------------------------------------------------------------------------
// entropy-stage helpers: canonical [N][C_a] symbols <-> tiled layout, escapes
// ---------------------------------------------------------------------------
__global__ void k_sym_to_tiled(const uint8_t *sym, uint32_t *sym32, int64_t N, int64_t N256, int Ca) {
  // one thread per (quad, rank)
  const int64_t nq = (N + 3) / 4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nq * Ca; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t qd = i / Ca;
    const int r = (int)(i - qd * Ca);
    uint32_t w = 0;
    for (int k = 0; k < 4; ++k) {
      const int64_t j = qd * 4 + k;
      const uint32_t s = j < N ? sym[(size_t)j * Ca + r] : 255u;
      w |= s << (8 * k);
    }
    sym32[((size_t)(r >> 6) * (N256 / 4) + qd) * 64 + (r & 63)] = w;
  }
}

__global__ void k_sym_from_tiled(const uint32_t *sym32, uint8_t *sym, int64_t N, int64_t N256, int Ca,
                                 const int32_t *status) {
  if (*status != 0) return;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < N * Ca; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t j = i / Ca;
    const int r = (int)(i - j * Ca);
    const uint32_t w = sym32[((size_t)(r >> 6) * (N256 / 4) + j / 4) * 64 + (r & 63)];
    sym[i] = (uint8_t)(w >> (8 * (j & 3)));
  }
}

// the caller's records into the raw list (the scan's sort leaves their
// ascending order as it is)
__global__ void k_load_esc(const uint32_t *esc, uint32_t n_esc, uint32_t *esc_raw, uint8_t *ws) {
  if (blockIdx.x == 0 && threadIdx.x == 0) ctrl_of(ws)->n_esc = n_esc;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < 2 * n_esc; i += gridDim.x * blockDim.x)
    esc_raw[i] = esc[i];
}

__global__ void k_copy_n_esc(const uint8_t *ws, uint32_t *n_esc_out, const int32_t *status) {
  *n_esc_out = *status == 0 ? reinterpret_cast<const Ctrl *>(ws)->n_esc : 0u;
}

unsigned grid_for(int64_t work, int per_block = 256, unsigned cap = 8192) {
  int64_t g = (work + per_block - 1) / per_block;
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(g, cap));
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
void launch_rans_encode(const EncodeArgs &a) {
  if (a.g.n_groups == 0) return;
  EncP P;
  P.tab = a.p->dev.tab;
  P.sym32 = reinterpret_cast<const uint32_t *>(a.ws + a.l.sym);
  P.scratch = reinterpret_cast<uint16_t *>(a.ws + a.l.scratch);
  P.gwords = reinterpret_cast<uint32_t *>(a.ws + a.l.gwords);
  P.N = a.g.N;
  P.N256 = a.g.N256;
  P.n_blk = a.g.n_blk;
  P.Ca = a.p->C_a;
  P.G = a.p->G;
  P.status = a.status;
  dim3 grid((unsigned)((a.g.n_blk + kEncWaves - 1) / kEncWaves), (unsigned)a.p->G);
  KernelTimer tm("rans_encode", a.s);
  hipLaunchKernelGGL(k_rans_encode, grid, dim3(kEncWaves * 64), 0, a.s, P);
}

void launch_scan_header(const EncodeArgs &a) {
  ScanP P;
  P.esc_raw = reinterpret_cast<uint32_t *>(a.ws + a.l.esc_raw);
  P.esc_sorted = reinterpret_cast<uint32_t *>(a.ws + a.l.esc_sorted);
  P.gwords = reinterpret_cast<const uint32_t *>(a.ws + a.l.gwords);
  P.goffs = reinterpret_cast<uint64_t *>(a.ws + a.l.goffs);
  P.ws = a.ws;
  P.stream = a.stream;
  P.capacity = a.capacity;
  P.stream_bytes = a.stream_bytes;
  P.status = a.status;
  P.n_groups = a.g.n_groups;
  P.esc_cap = a.g.esc_cap;
  P.kept_bytes = (uint64_t)a.g.n_kept * a.p->D * 2;
  P.T = (uint32_t)a.g.T;
  P.keep_head = (uint32_t)a.p->keep_head;
  P.keep_tail = (uint32_t)a.p->keep_tail;
  P.N = (uint32_t)a.g.N;
  P.n_coef = (uint32_t)a.p->C;
  P.Ca = (uint32_t)a.p->C_a;
  P.crc = a.p->crc;
  P.step_scale = a.p->step_scale;
  KernelTimer tm("scan", a.s);
  hipLaunchKernelGGL(k_scan_header, dim3(1), dim3(1024), 0, a.s, P);
}

void launch_pack(const EncodeArgs &a) {
  PackP P;
  P.scratch = reinterpret_cast<const uint16_t *>(a.ws + a.l.scratch);
  P.gwords = reinterpret_cast<const uint32_t *>(a.ws + a.l.gwords);
  P.goffs = reinterpret_cast<const uint64_t *>(a.ws + a.l.goffs);
  P.esc_sorted = reinterpret_cast<const uint32_t *>(a.ws + a.l.esc_sorted);
  P.ws = a.ws;
  P.stream = a.stream;
  P.n_groups = a.g.n_groups;
  P.status = a.status;
  const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>(a.g.n_groups, 65535));
  KernelTimer tm("pack", a.s);
  hipLaunchKernelGGL(k_pack, dim3(grid), dim3(256), 0, a.s, P);
}

void launch_parse(const DecodeArgs &a, bool with_rope) {
  ParseP P;
  P.stream = a.stream;
  P.size = a.stream_size;
  P.ws = a.ws;
  P.status = a.status;
  P.T = (uint32_t)a.g.T;
  P.keep_head = (uint32_t)a.p->keep_head;
  P.keep_tail = (uint32_t)a.p->keep_tail;
  P.N = (uint32_t)a.g.N;
  P.n_coef = (uint32_t)a.p->C;
  P.Ca = (uint32_t)a.p->C_a;
  P.crc = a.p->crc;
  P.n_groups = (uint32_t)a.g.n_groups;
  P.kept_bytes = (uint64_t)a.g.n_kept * a.p->D * 2;
  P.esc_rows = reinterpret_cast<uint32_t *>(a.ws + a.l.esc_rows);
  P.n_row_tiles = (uint32_t)a.g.n_mtiles;
  P.omega = a.p->dev.omega;
  P.rope_lo = reinterpret_cast<float2 *>(a.ws + a.l.rope_lo);
  P.rope_hi = reinterpret_cast<float2 *>(a.ws + a.l.rope_hi);
  P.rope_hi_n = a.g.rope_hi;
  const int64_t n_rope = with_rope ? (256 + a.g.rope_hi) * kHalf : 0;
  const unsigned rope_blocks = (unsigned)std::min<int64_t>((n_rope + 255) / 256, 4096);
  KernelTimer tm("parse", a.s);
  hipLaunchKernelGGL(k_parse, dim3(1 + rope_blocks), dim3(256), 0, a.s, P);
}

void launch_rans_decode(const DecodeArgs &a) {
  if (a.g.n_groups == 0) return;
  DecP P;
  P.tab = a.p->dev.tab;
  P.bucket = a.p->dev.bucket;
  P.stream = a.stream;
  P.ws = a.ws;
  P.esc_rows = reinterpret_cast<const uint32_t *>(a.ws + a.l.esc_rows);
  P.sym32 = reinterpret_cast<uint32_t *>(a.ws + a.l.sym);
  P.N = a.g.N;
  P.N256 = a.g.N256;
  P.n_blk = a.g.n_blk;
  P.Ca = a.p->C_a;
  P.G = a.p->G;
  P.status = a.status;
  dim3 grid((unsigned)((a.g.n_blk + kDecWaves - 1) / kDecWaves), (unsigned)a.p->G);
  KernelTimer tm("rans_decode", a.s);
  hipLaunchKernelGGL(k_rans_decode, grid, dim3(kDecWaves * 64), 0, a.s, P);
}

void launch_sym_to_tiled(const EncodeArgs &a, const uint8_t *sym) {
  if (a.g.N == 0 || a.p->C_a == 0) return;
  const int64_t work = (a.g.N + 3) / 4 * a.p->C_a;
  hipLaunchKernelGGL(k_sym_to_tiled, dim3(grid_for(work)), dim3(256), 0, a.s, sym,
                     reinterpret_cast<uint32_t *>(a.ws + a.l.sym), a.g.N, a.g.N256, a.p->C_a);
}

void launch_sym_from_tiled(const DecodeArgs &a, uint8_t *sym_out, uint32_t *n_esc_out) {
  if (a.g.N > 0 && a.p->C_a > 0) {
    hipLaunchKernelGGL(k_sym_from_tiled, dim3(grid_for(a.g.N * a.p->C_a)), dim3(256), 0, a.s,
                       reinterpret_cast<const uint32_t *>(a.ws + a.l.sym), sym_out, a.g.N, a.g.N256, a.p->C_a,
                       a.status);
  }
  if (n_esc_out) hipLaunchKernelGGL(k_copy_n_esc, dim3(1), dim3(1), 0, a.s, a.ws, n_esc_out, a.status);
}

void launch_load_esc(const EncodeArgs &a, const uint32_t *esc, uint32_t n_esc) {
  hipLaunchKernelGGL(k_load_esc, dim3(grid_for(2 * (int64_t)n_esc)), dim3(256), 0, a.s, esc, n_esc,
                     reinterpret_cast<uint32_t *>(a.ws + a.l.esc_raw), a.ws);
}

}  // namespace dckv
