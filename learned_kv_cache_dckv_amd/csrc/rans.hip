// Lossless stage of the DCKV codec on gfx950: interleaved 32-bit rANS over
// (256-token block, 64 active components) groups, the stream writer and the
// stream parser.
//
// Source: DCKV digest page ("DCKV: Learned Transform Coding of the Prompt KV
// Cache in Hybrid Language Models"), "How it works", Coding bullet: the
// integer codes go through an asymmetric-numeral-system coder whose symbol
// model is a discretised Laplace, and a code outside [-127, 127] leaves that
// coder and travels as a 64-bit record.  Coder parameters and layout are this
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
#include <type_traits>

#include "dckv_internal.h"

namespace dckv {
namespace {

constexpr int kEncWaves = 16;     // groups (waves) per encoder workgroup, one component group
constexpr int kDecWaves = 16;
constexpr int kWordBuf = 1024;    // u16 words cached per decoder wave

__device__ __forceinline__ void set_status(int32_t *st, int code) { atomicCAS(st, 0, code); }

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// A load through a global (address space 1) pointer.
template <class T>
__device__ __forceinline__ T gload(const T *p) {
  return *(const T __attribute__((address_space(1))) *)p;
}

// A 64 x 256 block of 32-bit table entries (components 64 g .. 64 g + 63 of a
// plan table [C_a][256]) into LDS transposed, entry (e, lane) at e * 64 +
// lane: a wave that reads one entry per lane, each lane its own component at
// its own index, then touches bank lane % 32 from every lane (two lanes per
// bank, the minimum), whatever the indices.  Columns past the group's n
// components are zero.  Piece pc (16 bytes) is entries 4 (pc / 64) .. + 3 of
// component pc % 64, so the 64 lanes of a wave write one LDS row each time,
// on consecutive banks.  Every thread issues its loads before its first LDS
// write, so the copy costs one memory latency.
template <int kThreads>
__device__ __forceinline__ void stage_tab(uint32_t *tab, const uint32_t *gtab, int g, int n) {
  constexpr int kPer = kLanes * 256 / 4 / kThreads;  // 16-byte pieces per thread
  static_assert(kPer * kThreads * 4 == kLanes * 256, "whole pieces");
  const u32x4 *src = reinterpret_cast<const u32x4 *>(gtab + (size_t)kLanes * g * 256);
  u32x4 v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int pc = threadIdx.x + i * kThreads;
    const int c = pc & 63, q = pc >> 6;
    // every load is issued (columns past n read column 0) before any is used
    v[i] = gload(src + (c < n ? c : 0) * 64 + q);
    if (c >= n) v[i] = u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int pc = threadIdx.x + i * kThreads;
    uint32_t *d = tab + (pc >> 6) * 4 * kLanes + (pc & 63);
    d[0] = v[i].x;
    d[kLanes] = v[i].y;
    d[2 * kLanes] = v[i].z;
    d[3 * kLanes] = v[i].w;
  }
}

__device__ __forceinline__ Ctrl *ctrl_of(uint8_t *ws) { return reinterpret_cast<Ctrl *>(ws); }

struct EncP {
  const uint32_t *tab;     // [C_a][256]
  const float *rcp;        // [C_a][256] scaled reciprocals of f
  const uint32_t *sym32;   // tiled symbols
  uint16_t *scratch;       // [n_groups][64 * 258]
  uint32_t *gwords;        // [n_groups]
  int64_t N, N256, n_blk;
  int Ca, G;
  const int32_t *status;
};

// The table entries and the reciprocals of components 64 g .. 64 g + 63 into
// LDS as pairs (entry, reciprocal), pair (e, lane) at e * 64 + lane: a wave
// reads every lane's pair with one 8-byte LDS read, and the bank depends on
// the lane alone, as in stage_tab().  Columns past n are zero.
template <int kThreads>
__device__ __forceinline__ void stage_pairs(u32x2 *pr, const uint32_t *gtab, const uint32_t *grcp, int g, int n) {
  constexpr int kPer = kLanes * 256 / 4 / kThreads;
  static_assert(kPer * kThreads * 4 == kLanes * 256, "whole pieces");
  const u32x4 *st = reinterpret_cast<const u32x4 *>(gtab + (size_t)kLanes * g * 256);
  const u32x4 *sr = reinterpret_cast<const u32x4 *>(grcp + (size_t)kLanes * g * 256);
  u32x4 a[kPer], b[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int pc = threadIdx.x + i * kThreads;
    const int c = pc & 63, q = pc >> 6;
    // every load is issued (columns past n read column 0) before any is used
    const int cc = c < n ? c : 0;
    a[i] = gload(st + cc * 64 + q);
    b[i] = gload(sr + cc * 64 + q);
    if (c >= n) a[i] = b[i] = u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int pc = threadIdx.x + i * kThreads;
    u32x2 *d = pr + (pc >> 6) * 4 * kLanes + (pc & 63);
    d[0] = u32x2{a[i].x, b[i].x};
    d[kLanes] = u32x2{a[i].y, b[i].y};
    d[2 * kLanes] = u32x2{a[i].z, b[i].z};
    d[3 * kLanes] = u32x2{a[i].w, b[i].w};
  }
}

// Workgroup w of a request codes component group g = w / nch of the blocks
// 16 (w % nch) .. + 15 (one wave each), nch = ceil(n_blk / 16).
__global__ __launch_bounds__(kEncWaves * 64) void k_rans_encode(const Batch<EncP> B) {
  __shared__ u32x2 pairs[256 * kLanes];  // [symbol][lane]: (f | cum << 16, fp32 bits of the scaled 1/f)
  const int ri = batch_req(B, blockIdx.x);
  const EncP &P = B.r[ri];
  const uint32_t nch_w = (uint32_t)((P.n_blk + kEncWaves - 1) / kEncWaves);
  const uint32_t local = blockIdx.x - B.start[ri];
  const int g = (int)(local / nch_w);
  const int chunk = (int)(local - (uint32_t)g * nch_w);
  const int n = min(kLanes, P.Ca - kLanes * g);
  stage_pairs<kEncWaves * 64>(pairs, P.tab, reinterpret_cast<const uint32_t *>(P.rcp), g, n);
  __syncthreads();
  if (*P.status != 0) return;
  // the wave's block, its length and quad count are wave-uniform (scalar
  // registers, scalar branches)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t b = (int64_t)chunk * kEncWaves + wave;
  if (b >= P.n_blk) return;
  const int Lb = (int)min<int64_t>(kBlock, P.N - kBlock * b);
  const int64_t gid = b * P.G + g;
  const uint32_t *sw = P.sym32 + ((size_t)g * (P.N256 / 4) + (size_t)b * 64) * 64 + lane;
  uint16_t *out = P.scratch + (size_t)gid * (kLanes * (kBlock + 2));
  // the group's words go through a buffer resource over its scratch slot; a
  // lane that emits nothing stores to an offset past the range, which the
  // hardware drops, so no step changes the execution mask
  constexpr uint32_t kSlotWords = kLanes * (kBlock + 2), kSlotBytes = 2 * kSlotWords;
  constexpr int kDrop = 1 << 30;
  const rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(out, (short)0, (int)kSlotBytes, 0x00020000);
  const bool lane_ok = lane < n;
  // Escapes code as the identity: table entry 255 is f = 2^15, cum = 0, so
  // the state never emits and x / f * 2^15 + x % f = x.  Lanes past C_a code
  // escapes only, through lane 0's table row.
  const u32x2 *mypair = pairs + (lane_ok ? lane : 0);
  uint32_t x = kL;
  uint32_t cnt = 0;
  // One coding step of the pair (e, rf) = (f | cum << 16, scaled 1/f).
  // The lanes whose state is >= f 2^17 first emit their low 16 bits.  The
  // coder pushes a step's words in descending lane order and the stream holds
  // the pushes reversed, so the slot is filled from its top down: the step's
  // words go below those already there, in ascending lane order, and the
  // group's words end up in stream order at the top of the slot.
  // q0 = trunc(fp32(x) rf) is floor(x / f) or one less (the reciprocal is
  // scaled down so that the fp32 roundings never push it above), so
  // x' = q M + (x - q f) + cum = (q0 << 15) + r0 + cum, plus M - f when
  // r0 = x - q0 f is still >= f.
  auto enc = [&](u32x2 te) {
    const uint32_t e = te.x, f = e & 0xFFFFu;
    const float rf = __uint_as_float(te.y);
    const bool emit = (x >> 17) >= f;  // x >= f 2^17 (f = 2^15 never emits)
    const uint64_t mask = __ballot(emit);
    const uint32_t tot = (uint32_t)__popcll(mask);
    const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
    // all-ones on the emitting lanes, as a value (the selections below stay
    // arithmetic: no branch and no change of the execution mask)
    uint32_t sel = emit ? 0xFFFFFFFFu : 0u;
    asm volatile("" : "+v"(sel));
    const uint32_t voff = ((2u * (kSlotWords - cnt - tot) + 2u * below) & sel) | ((uint32_t)kDrop & ~sel);
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)x, wr, (int)voff, 0, 0);
    x >>= sel & 16u;
    cnt += tot;
    const uint32_t q0 = (uint32_t)((float)x * rf);
    const uint32_t r0 = x - __umul24(q0, f);
    const uint32_t xn = (q0 << kPrecBits) + r0 + (e >> 16);
    x = xn + (r0 >= f ? kM - f : 0u);
  };
  // Quads (symbol words of four rows) are coded last to first, in chunks of
  // eight whose words are loaded one chunk ahead.  Quads past the block's
  // last code as escapes (the identity), as do the rows past the block in its
  // last quad, so every chunk is whole and the loop has no per-lane branch.
  const int nq = (Lb + 3) >> 2;
  const int nch = (nq + 7) >> 3;
  const uint32_t tail = (Lb & 3) ? 0xFFFFFFFFu << (8 * (Lb & 3)) : 0u;
  uint32_t wq[8], wn[8];
  auto load_chunk = [&](int ch, uint32_t (&w)[8]) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int qd = ch * 8 + u;
      const uint32_t v = gload(sw + (size_t)qd * 64);
      w[u] = !lane_ok || qd >= nq ? 0xFFFFFFFFu : (qd == nq - 1 ? v | tail : v);
    }
  };
  // the four pairs of a quad's symbols; a quad's pairs are read while the
  // quad before it in coding order is coded, so a step never waits on LDS
  auto fetch = [&](uint32_t w, u32x2 (&t)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) t[k] = mypair[((w >> (8 * k)) & 0xFFu) * kLanes];
  };
  u32x2 ec[4], en[4];
  load_chunk(nch - 1, wn);
  fetch(wn[7], ec);
#pragma unroll 1
  for (int ch = nch - 1; ch >= 0; --ch) {
#pragma unroll
    for (int u = 0; u < 8; ++u) wq[u] = wn[u];
    if (ch > 0) load_chunk(ch - 1, wn);
#pragma unroll
    for (int u = 7; u >= 0; --u) {
      // the next quad in coding order: u - 1 of this chunk, or quad 7 of the
      // next chunk
      if (u > 0)
        fetch(wq[u - 1], en);
      else if (ch > 0)
        fetch(wn[7], en);
#pragma unroll
      for (int k = 3; k >= 0; --k) enc(ec[k]);
#pragma unroll
      for (int k = 0; k < 4; ++k) ec[k] = en[k];
    }
  }
  // the final states come first in the stream: lane l's low and high halves
  // at words 2 l and 2 l + 1
  if (lane_ok) {
    const uint32_t pos = kSlotWords - cnt - 2u * (uint32_t)n + 2u * (uint32_t)lane;
    out[pos] = (uint16_t)(x & 0xFFFFu);
    out[pos + 1] = (uint16_t)(x >> 16);
  }
  if (lane == 0) P.gwords[gid] = cnt + 2u * (uint32_t)n;
}

// ---------------------------------------------------------------------------
// group-size scan, group offsets, header, final size
// ---------------------------------------------------------------------------
// Escapes (codes beyond +-127, 64 bits each) are found out of order by the
// quantiser tiles; the stream stores them by ascending flat index
// j * C_a + rank, so the scan's workgroup first sorts the (usually few)
// records: up to one record per thread by counting the smaller keys, beyond
// that with a bitonic network, in LDS up to kSortLds records, else in place
// in global memory.
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
  if (n <= blockDim.x) {
    // each record's place is the number of records before it in (flat
    // index, arrival) order (the flat indices of a valid encode are distinct;
    // arrival order only keeps the places distinct whatever the input): one
    // pass, one thread per record, no barriers
    if (threadIdx.x < n) {
      const unsigned long long v = a[threadIdx.x];
      const unsigned long long key = v >> 32;
      uint32_t pos = 0;
      for (uint32_t j = 0; j < n; ++j) {
        const unsigned long long kj = a[j] >> 32;
        pos += (kj < key || (kj == key && j < threadIdx.x)) ? 1u : 0u;
      }
      esc_sorted[2 * pos] = (uint32_t)(v >> 32);
      esc_sorted[2 * pos + 1] = (uint32_t)v;
    }
    return;
  }
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

// One workgroup per request.
constexpr int kScanChunk = 4096;
__global__ __launch_bounds__(1024) void k_scan_header(const Batch<ScanP> B) {
  const ScanP &P = B.r[batch_req(B, blockIdx.x)];
  __shared__ uint64_t part[16];
  __shared__ uint64_t sbuf[kScanChunk];
  __shared__ unsigned long long keys[kSortLds];
  const int t = threadIdx.x;
  if (*P.status == 0) sort_escapes(P.ws, P.esc_raw, P.esc_sorted, P.esc_cap, keys);
  __syncthreads();
  // group word offsets: chunks of 4,096 groups go through LDS, so that the
  // loads and stores are coalesced and each thread scans 4 consecutive sizes
  const int64_t ng = P.n_groups;
  const int lane = t & 63, wv = t >> 6;
  uint64_t carry = 0;
  for (int64_t c0 = 0; c0 < ng; c0 += kScanChunk) {
    const int64_t m = min<int64_t>(kScanChunk, ng - c0);
#pragma unroll
    for (int u = 0; u < kScanChunk / 1024; ++u) {
      const int64_t i = t + 1024 * u;
      sbuf[i] = i < m ? P.gwords[c0 + i] : 0u;
    }
    __syncthreads();
    const uint64_t e0 = sbuf[4 * t], e1 = sbuf[4 * t + 1], e2 = sbuf[4 * t + 2], e3 = sbuf[4 * t + 3];
    const uint64_t s = e0 + e1 + e2 + e3;
    // inclusive scan: within each wave by shuffles, then the 16 wave totals
    uint64_t incl = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint64_t v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    if (lane == 63) part[wv] = incl;
    __syncthreads();
    uint64_t before = 0, all = 0;
    for (int w = 0; w < 16; ++w) {
      if (w < wv) before += part[w];
      all += part[w];
    }
    const uint64_t ex = carry + before + incl - s;
    sbuf[4 * t] = ex;
    sbuf[4 * t + 1] = ex + e0;
    sbuf[4 * t + 2] = ex + e0 + e1;
    sbuf[4 * t + 3] = ex + e0 + e1 + e2;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kScanChunk / 1024; ++u) {
      const int64_t i = t + 1024 * u;
      if (i < m) P.goffs[c0 + i] = sbuf[i];
    }
    carry += all;
    __syncthreads();  // sbuf and part are reused by the next chunk
  }
  const uint64_t total_words = carry;
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

// Workgroup b of a request copies group b (the top W words of its slot) to
// its offset (256 words per pass, coalesced both ways); the request's
// workgroups also copy its escape records, in strides.
__global__ __launch_bounds__(256) void k_pack(const Batch<PackP> B) {
  const int ri = batch_req(B, blockIdx.x);
  const PackP &P = B.r[ri];
  const uint32_t local = blockIdx.x - B.start[ri], cnt = B.start[ri + 1] - B.start[ri];
  // the status, the control words and the group's size and offset are read
  // together (all lie in the workspace whatever the status)
  const Ctrl *ct = reinterpret_cast<const Ctrl *>(P.ws);
  const int64_t gid = local;
  const bool has_group = gid < P.n_groups;
  const int32_t st = *P.status;
  const uint64_t rans_off = ct->rans_off, esc_off = ct->esc_off;
  const uint32_t n_esc = ct->n_esc;
  const uint32_t W = has_group ? P.gwords[gid] : 0u;
  const uint64_t goff = has_group ? P.goffs[gid] : 0u;
  if (st != 0) return;
  if (has_group) {
    const uint16_t *src = P.scratch + (size_t)(gid + 1) * (kLanes * (kBlock + 2)) - W;
    uint16_t *dst = reinterpret_cast<uint16_t *>(P.stream + rans_off) + goff;
    // four words per thread per pass, loaded before any is stored
    constexpr uint32_t kU = 4;
    for (uint32_t k0 = threadIdx.x; k0 < W; k0 += kU * blockDim.x) {
      uint16_t v[kU];
#pragma unroll
      for (uint32_t u = 0; u < kU; ++u) {
        const uint32_t k = k0 + u * blockDim.x;
        if (k < W) v[u] = src[k];
      }
#pragma unroll
      for (uint32_t u = 0; u < kU; ++u) {
        const uint32_t k = k0 + u * blockDim.x;
        if (k < W) dst[k] = v[u];
      }
    }
  }
  uint32_t *e = reinterpret_cast<uint32_t *>(P.stream + esc_off);
  for (uint32_t i = local * blockDim.x + threadIdx.x; i < n_esc; i += cnt * blockDim.x) {
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

// Workgroup 0 of a request checks its stream; the others (if any) build its
// RoPE tables.
__global__ __launch_bounds__(256) void k_parse(const Batch<ParseP> B) {
  const int ri = batch_req(B, blockIdx.x);
  const ParseP &P = B.r[ri];
  const uint32_t local = blockIdx.x - B.start[ri], cnt = B.start[ri + 1] - B.start[ri];
  __shared__ int bad;
  __shared__ int plan_bad;
  __shared__ uint64_t s_esc_off, s_rans_off, s_rans_bytes;
  __shared__ uint32_t s_n_esc;
  const int t = threadIdx.x;
  if (local > 0) {
    const int64_t n = (256 + P.rope_hi_n) * kHalf;
    for (int64_t i = (int64_t)(local - 1) * blockDim.x + t; i < n; i += (int64_t)(cnt - 1) * blockDim.x) {
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
    uint32_t h[kHeaderBytes / 4];
    if (P.size >= (uint64_t)kHeaderBytes) {
      // all header words in flight at once
#pragma unroll
      for (int i = 0; i < kHeaderBytes / 4; ++i) h[i] = reinterpret_cast<const uint32_t *>(P.stream)[i];
    }
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
    // thread t checks the offsets of groups [16 t, 16 t + 16) of each pass:
    // 17 loads issued together (indices clamped to the last entry, which
    // exists), then the 16 pairs inside the request
    constexpr uint32_t kOffRun = 16;
    for (uint32_t g0 = t * kOffRun; g0 < P.n_groups; g0 += blockDim.x * kOffRun) {
      uint32_t o[kOffRun + 1];
#pragma unroll
      for (uint32_t j = 0; j <= kOffRun; ++j) o[j] = offs[min(g0 + j, P.n_groups)];
#pragma unroll
      for (uint32_t j = 0; j < kOffRun; ++j)
        if (g0 + j < P.n_groups && (o[j + 1] < o[j] || (o[j] & 1) || (o[j + 1] & 1))) my_bad = 1;
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
  const uint32_t *bucket;
  // fused dequantisation (a plan without dropped components): the decoder
  // writes yhat_b itself; the odd row that ends each block but the last is
  // finished by k_dequant_fix from the four halo arrays [n_blk][C]
  int fuse;
  const float *mtab;         // [vocab][C] embedding means
  const int32_t *tok;
  const float *step, *nbr;
  uint16_t *yhat_b;          // [NM][C]
  float *hm, *hq, *hl, *hr;  // the pending row's mean and code, its left neighbour; each block's first yhat
  int keep_head, vocab;
  const uint8_t *stream;
  const uint8_t *ws;
  const uint32_t *esc_rows;  // [blocks][2]: index range of each block's escape records (from the parser)
  uint32_t *sym32;
  int64_t N, N256, n_blk;
  int Ca, G;
  int32_t *status;
};

// The LDS address of a shared array, and a shared-memory object at an LDS
// address.
template <class T>
__device__ __forceinline__ uint32_t lds_addr(T *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
template <class T>
__device__ __forceinline__ const __attribute__((address_space(3))) T *lds_at(uint32_t a) {
  return (const __attribute__((address_space(3))) T *)(uintptr_t)a;
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Lane q's copy of a per-lane 64-bit value (q wave-uniform).
__device__ __forceinline__ uint64_t readlane64(uint64_t v, int q) {
  return (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, q) |
         ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), q) << 32);
}

// The symbols of one wave's rows: step i pops the symbol of row i from each
// lane's state, then renormalises the lanes that need it with the next words
// of the interleaved stream, in lane order.  The symbol of a slot comes from
// its bucket: lo, or lo + 1 from the bucket's split slot on; only buckets of
// three or more symbols take a binary search over the cumulative table (rare:
// a wave enters it only while one of its lanes sits in such a bucket).
// kPlain: every lane is a coded component and the block has no escapes, so no
// lane is ever skipped; otherwise lane l of row 4 q + k is skipped when bit l
// of lane q's esc[k] is set.  A step has no branch of its own: every lane
// reads a word of the window and keeps it only if it renormalises.  The window
// slides (before a quad) when the quad could read past it; it is read modulo
// its size, so a corrupt stream reads words of the window, never past it, and
// ends with ptr != W or a final state != L, which the caller reports.
// quad.template run<PH>(q, s0, s1, s2, s3, rows) takes the symbols of rows
// 4 q .. 4 q + rows - 1 (rows past the block read as escapes);
// quad.template pre<PH>(q) runs before the quad's steps (prefetches).  PH is
// q mod 3 for whole quads, a constant at every call: the quad loop is unrolled
// by three, so a functor can rotate three buffers without copying them.  The
// partial quad runs with PH = 0 after quad.to_phase0(q mod 3).
template <bool kPlain, class Fill, class Quad>
__device__ __forceinline__ void decode_rows(uint32_t &x, uint32_t &ptr, uint32_t &base, uint32_t W, int Lb, int lane,
                                            bool lane_ok, bool has_esc, const uint64_t (&esc)[4],
                                            const uint32_t *mytab, const uint32_t *mybkt, uint32_t bkt_lane, uint32_t wofs,
                                            Fill &&fill, Quad &&quad) {
  // emask: the row's escaped lanes (bit l set: lane l is skipped)
  auto step = [&](uint64_t emask) -> uint32_t {
    bool act = true;
    if (!kPlain) act = lane_ok && !((emask >> lane) & 1ull);
    const uint32_t slot = x & (kM - 1u);
    // bucket row (slot >> 7) of 256 bytes, this lane's word in it (the mask
    // is kept apart from the shift-add, one instruction each)
    uint32_t brow = x & 0x7F80u;
    asm volatile("" : "+v"(brow));
    const uint32_t be = *lds_at<uint32_t>((brow << 1) + bkt_lane);
    const uint32_t split = be >> 16;
    uint32_t s = (be & 0xFFu) + (slot >= split ? 1u : 0u);
    const bool srch = act && split == kSplitSearch;
    if (__builtin_expect(__ballot(srch) != 0ull, 0)) {
      // candidates lo .. the first symbol of the next bucket
      const uint32_t bi = slot >> kBucketShift;
      uint32_t lo = s, hi = s;
      if (srch) hi = bi + 1 < (uint32_t)kBuckets ? (uint32_t)(mybkt[(bi + 1) * kLanes] & 0xFFu) : (uint32_t)(kNSym - 1);
      while (__ballot(lo < hi)) {
        const uint32_t mid = (lo + hi + 1) >> 1;
        const bool up = (mytab[mid * kLanes] >> 16) <= slot;
        const bool open = lo < hi;
        lo = open && up ? mid : lo;
        hi = open && !up ? mid - 1 : hi;
      }
      s = lo;
    }
    const uint32_t e = mytab[s * kLanes];
    // f * (x >> 15) < 2^32: f <= 2^15 and x >> 15 < 2^17 (24-bit multiply)
    const uint32_t xd = __umul24(e & 0xFFFFu, x >> kPrecBits) + slot - (e >> 16);
    x = act ? xd : x;
    const bool need = act && x < kL;
    const uint64_t mask = __ballot(need);
    const uint32_t before = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
    // the word window is 2 KiB-aligned: its offset is ORed in
    uint32_t wv = *lds_at<uint16_t>(((2u * (ptr - base) + 2u * before) & (2u * kWordBuf - 2u)) | wofs);
    asm volatile("" : "+v"(wv));
    x = need ? (x << 16) | wv : x;
    ptr += (uint32_t)__popcll(mask);
    return act ? s : (uint32_t)kEsc;
  };
  // the escaped lanes of row 4 q + k (lane q's esc[k]; k is a constant at
  // every call, so esc stays in registers)
  auto em = [&](int q, int k) -> uint64_t {
    return (!kPlain && has_esc) ? readlane64(esc[k], q) : 0ull;
  };
  // a quad takes at most 4 * 64 words: slide the window to ptr first when
  // they could reach past it (and the stream goes on past it)
  auto slide = [&]() {
    if (ptr + 4u * kLanes > base + kWordBuf && base + kWordBuf < W) {
      base = ptr;
      fill(base);
    }
  };
  auto whole = [&](int q, auto ph) __attribute__((always_inline)) {
    constexpr int PH = decltype(ph)::value;
    slide();
    quad.template pre<PH>(q);
    const uint32_t s0 = step(em(q, 0)), s1 = step(em(q, 1)), s2 = step(em(q, 2)), s3 = step(em(q, 3));
    quad.template run<PH>(q, s0, s1, s2, s3, 4);
  };
  // the last, partial quad: rows past the block read as escapes
  auto part = [&](int q, int r, auto ph) __attribute__((always_inline)) {
    constexpr int PH = decltype(ph)::value;
    slide();
    quad.template pre<PH>(q);
    const uint32_t s0 = step(em(q, 0));
    const uint32_t s1 = r > 1 ? step(em(q, 1)) : (uint32_t)kEsc;
    const uint32_t s2 = r > 2 ? step(em(q, 2)) : (uint32_t)kEsc;
    quad.template run<PH>(q, s0, s1, s2, (uint32_t)kEsc, r);
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  const int nq = Lb >> 2;
  int q = 0;
#pragma unroll 1
  for (; q + 3 <= nq; q += 3) {
    whole(q, P0{});
    whole(q + 1, P1{});
    whole(q + 2, P2{});
  }
  // at most two whole quads left (phases 0 and 1), then the partial one
  if (q < nq) whole(q, P0{});
  if (q + 1 < nq) whole(q + 1, P1{});
  if (Lb & 3) {
    // the partial quad's phase is nq - q (0, 1 or 2): its buffer moves to
    // phase 0 by value (a buffer index that is not a constant would put the
    // functor in scratch memory)
    quad.to_phase0(nq - q);
    part(nq, Lb & 3, P0{});
  }
}

// The decoder's per-quad work on symbols only: the symbol words.
struct SymOnly {
  uint32_t *sout;
  bool ok;
  __device__ __forceinline__ void to_phase0(int) {}
  template <int PH>
  __device__ __forceinline__ void pre(int) {}
  template <int PH>
  __device__ __forceinline__ void run(int q, uint32_t s0, uint32_t s1, uint32_t s2, uint32_t s3, int) {
    if (ok) sout[(size_t)q * 64] = s0 | (s1 << 8) | (s2 << 16) | (s3 << 24);
  }
};

// The decoder's per-quad work with the dequantisation fused (see
// k_rans_decode).
struct Fused {
  const float *mcol;  // mtab + c
  uint16_t *ycol;     // yhat_b + c
  uint32_t tk[4];     // token ids of rows 4 l .. 4 l + 3 (lane l)
  const uint32_t *erec;
  uint32_t elo, ehi;
  int32_t *status;
  int64_t j0, N, n_blk, b;
  int Ca, c;
  float st, a;
  float m[3][4];      // means of quad q in m[q mod 3] (loaded two quads ahead)
  float yl, mp, qp;   // the pending odd row: left neighbour, mean, code
  __device__ __forceinline__ float mean(int qq, int k) const {
    const uint32_t id = (uint32_t)__builtin_amdgcn_readlane((int)tk[k], qq);
    return gload(mcol + (size_t)id * kC);
  }
  // quads 0 and 1 before the loop; quad q + 2 at quad q (buffer (q + 2) mod 3)
  __device__ __forceinline__ void prime() {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      m[0][k] = mean(0, k);
      m[1][k] = mean(1, k);
    }
  }
  __device__ __forceinline__ void to_phase0(int ph) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float v0 = m[0][k], v1 = m[1][k], v2 = m[2][k];
      // values, not addresses: a select of addresses is a dynamic index
      asm volatile("" : "+v"(v0), "+v"(v1), "+v"(v2));
      m[0][k] = ph == 0 ? v0 : ph == 1 ? v1 : v2;
    }
  }
  template <int PH>
  __device__ __forceinline__ void pre(int q) {
    constexpr int B2 = (PH + 2) % 3;
    if (q + 2 < kLanes) {
#pragma unroll
      for (int k = 0; k < 4; ++k) m[B2][k] = mean(q + 2, k);
    }
  }
  // the code of escaped row j: its record among the block's (ascending flat)
  __device__ __forceinline__ float esc_code(int64_t j) const {
    const uint32_t flat = (uint32_t)j * (uint32_t)Ca + (uint32_t)c;
    uint32_t lo = elo, hi = ehi;
    while (lo < hi) {
      const uint32_t mid = (lo + hi) >> 1;
      if (gload(erec + 2 * mid) < flat) lo = mid + 1; else hi = mid;
    }
    if (lo < ehi && gload(erec + 2 * lo) == flat) return (float)(int)gload(erec + 2 * lo + 1);
    set_status(status, DCKV_ECORRUPT);
    return 0.f;
  }
  __device__ __forceinline__ void put(int64_t j, float y) { ycol[(size_t)j * kC] = __builtin_bit_cast(uint16_t, (__bf16)y); }
  template <int PH>
  __device__ __forceinline__ void run(int q, uint32_t s0, uint32_t s1, uint32_t s2, uint32_t s3, int rows) {
    const float(&mq)[4] = m[PH];
    const int64_t j = j0 + 4 * q;
    const uint32_t sy[4] = {s0, s1, s2, s3};
    float qv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      qv[k] = (float)((int)sy[k] - 127);
      const bool e = sy[k] == (uint32_t)kEsc && k < rows;
      if (__builtin_expect(__ballot(e) != 0ull, 0))
        if (e) qv[k] = esc_code(j + k);
    }
    const float y0 = mq[0] + qv[0] * st;
    if (q > 0) put(j - 1, mp + a * (yl + y0) + qp * st);
    else if (b > 0) hr_store(y0);
    put(j, y0);
    if (rows > 1) {
      const float y2 = rows > 2 ? mq[2] + qv[2] * st : 0.f;
      put(j + 1, mq[1] + a * (y0 + y2) + qv[1] * st);
      if (rows > 2) put(j + 2, y2);
      yl = y2;
    }
    mp = mq[3];
    qp = qv[3];
  }
  float *hr_ptr;
  __device__ __forceinline__ void hr_store(float y0) { *hr_ptr = y0; }
};

// Workgroup w of a request decodes component group g = w / nch of the blocks
// 16 (w % nch) .. + 15 (one wave each), nch = ceil(n_blk / 16).
__global__ __launch_bounds__(kDecWaves * 64) void k_rans_decode(const Batch<DecP> B) {
  const int ri = batch_req(B, blockIdx.x);
  const DecP &P = B.r[ri];
  const uint32_t nch_w = (uint32_t)((P.n_blk + kDecWaves - 1) / kDecWaves);
  const uint32_t local = blockIdx.x - B.start[ri];
  const int g = (int)(local / nch_w);
  const int chunk = (int)(local - (uint32_t)g * nch_w);
  __shared__ uint32_t tab[256 * kLanes];        // [symbol][lane]: f | cum << 16
  __shared__ uint32_t bkt[kBuckets * kLanes];    // [bucket][lane]: lo | split << 16
  __shared__ __attribute__((aligned(2048))) uint16_t wbuf[kDecWaves][kWordBuf];
  static_assert(kBuckets == 256, "bucket rows are staged like the tables");
  const int n = min(kLanes, P.Ca - kLanes * g);
  stage_tab<kDecWaves * 64>(tab, P.tab, g, n);
  stage_tab<kDecWaves * 64>(bkt, P.bucket, g, n);
  __syncthreads();
  if (*P.status != 0) return;
  // per-wave values are kept in scalar registers: the step loop is uniform,
  // and lanes that decode nothing at a step take the same path with their
  // results discarded
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t b = (int64_t)chunk * kDecWaves + wave;
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
  // the group's words through a buffer resource of W words: loads past the
  // end return zero, so a window fill issues all its loads at once
  const rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(wsrc), (short)0, (int)(2u * W),
                                                      0x00020000);
  auto fill = [&](uint32_t from) {
    uint16_t v[kWordBuf / 64];
    wave_sync_lds();
#pragma unroll
    for (int i = 0; i < kWordBuf / 64; ++i)
      v[i] = __builtin_amdgcn_raw_buffer_load_b16(wr, (int)(2u * (from + (uint32_t)lane + 64u * i)), 0, 0);
#pragma unroll
    for (int i = 0; i < kWordBuf / 64; ++i) wb[lane + 64 * i] = v[i];
    wave_sync_lds();
  };
  // escape positions of this group: a bitmap of the block's 256 rows, built
  // in the word buffer (2 KiB) and then held in registers, rows 4 l .. 4 l + 3
  // by lane l
  uint64_t esc[4] = {0ull, 0ull, 0ull, 0ull};
  bool has_esc = false;
  {
    const uint32_t *erec = reinterpret_cast<const uint32_t *>(P.stream + ct->esc_off);
    // the block's records, as the parser found them (a block is 256 rows)
    const uint32_t lo = __builtin_amdgcn_readfirstlane(gload(P.esc_rows + 2 * b));
    const uint32_t lo2 = __builtin_amdgcn_readfirstlane(gload(P.esc_rows + 2 * b + 1));
    if (lo2 > lo) {
      has_esc = true;
      unsigned long long *eb = reinterpret_cast<unsigned long long *>(wb);
      static_assert(kWordBuf * 2 >= kBlock * 8, "the bitmap fits in the word buffer");
      for (int i = lane; i < kBlock; i += 64) eb[i] = 0ull;
      wave_sync_lds();
      for (uint32_t e = lo + lane; e < lo2; e += 64) {
        const uint64_t f = erec[2 * e];
        const uint64_t jj = f / (uint64_t)P.Ca;
        const int r = (int)(f - jj * (uint64_t)P.Ca);
        if (r >= kLanes * g && r < kLanes * g + n)
          atomicOr(&eb[(int)(jj - (uint64_t)kBlock * b)], 1ull << (r - kLanes * g));
      }
      wave_sync_lds();
#pragma unroll
      for (int k = 0; k < 4; ++k) esc[k] = eb[4 * lane + k];
    }
  }
  // word window [base, base + kWordBuf)
  uint32_t base = 0;
  fill(0);
  uint32_t x = kL;
  if (lane_ok) x = (uint32_t)wb[2 * lane] | ((uint32_t)wb[2 * lane + 1] << 16);
  uint32_t ptr = 2u * (uint32_t)n;
  const uint32_t *mytab = tab + lane;
  const uint32_t *mybkt = bkt + lane;
  const uint32_t bkt_lane = lds_addr(mybkt);
  uint32_t *sout = P.sym32 + ((size_t)g * (P.N256 / 4) + (size_t)b * 64) * 64 + lane;
  uint32_t wofs = lds_addr(wb);
  asm volatile("" : "+v"(wofs));  // in a VGPR: a window address is then one and-or
  if (!P.fuse) {
    if (!has_esc && n == kLanes)
      decode_rows<true>(x, ptr, base, W, Lb, lane, true, false, esc, mytab, mybkt, bkt_lane, wofs, fill,
                        SymOnly{sout, true});
    else
      decode_rows<false>(x, ptr, base, W, Lb, lane, lane_ok, has_esc, esc, mytab, mybkt, bkt_lane, wofs, fill,
                         SymOnly{sout, lane_ok});
  } else {
    // Fused dequantisation (every component coded: lane = component = mean
    // table column c).  Row j of the block: yhat = mu + q step on even rows;
    // an odd row waits for the next even one, mu + a (yhat_{j-1} + yhat_{j+1})
    // + q step; the odd row past the request's end takes 0 on the right.  The
    // block's last odd row, unless it is the request's last, goes to the halo
    // (mean, code, left neighbour) with each block's first yhat, for
    // k_dequant_fix.  Means: lane l holds the token ids of rows 4 l .. 4 l + 3
    // (ids out of range set EINVAL and read as 0); a quad's means are loaded
    // two quads ahead.  Escaped codes come from the block's records.  The
    // symbols themselves are not stored: nothing after this reads them.
    const int c = kLanes * g + lane;
    const int64_t j0 = (int64_t)kBlock * b;
    uint32_t tk[4];
    {
      bool badtok = false;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t j = j0 + 4 * lane + k;
        int v = j < P.N ? gload(P.tok + P.keep_head + j) : 0;
        if (v < 0 || v >= P.vocab) {
          badtok = true;
          v = 0;
        }
        tk[k] = (uint32_t)v;
      }
      if (__ballot(badtok) != 0ull && lane == 0) set_status(P.status, DCKV_EINVAL);
    }
    const uint32_t *erec = reinterpret_cast<const uint32_t *>(P.stream + ct->esc_off);
    const uint32_t elo = __builtin_amdgcn_readfirstlane(gload(P.esc_rows + 2 * b));
    const uint32_t ehi = __builtin_amdgcn_readfirstlane(gload(P.esc_rows + 2 * b + 1));
    Fused fz;
    fz.mcol = P.mtab + c;
    fz.ycol = P.yhat_b + c;
#pragma unroll
    for (int k = 0; k < 4; ++k) fz.tk[k] = tk[k];
    fz.erec = erec;
    fz.elo = elo;
    fz.ehi = ehi;
    fz.status = P.status;
    fz.j0 = j0;
    fz.N = P.N;
    fz.n_blk = P.n_blk;
    fz.b = b;
    fz.Ca = P.Ca;
    fz.c = c;
    fz.st = gload(P.step + c);
    fz.a = gload(P.nbr + c);
    fz.yl = fz.mp = fz.qp = 0.f;
    fz.hr_ptr = P.hr + (size_t)b * kC + c;
    fz.prime();
    if (!has_esc)
      decode_rows<true>(x, ptr, base, W, Lb, lane, true, false, esc, mytab, mybkt, bkt_lane, wofs, fill, fz);
    else
      decode_rows<false>(x, ptr, base, W, Lb, lane, true, has_esc, esc, mytab, mybkt, bkt_lane, wofs, fill, fz);
    // the block's last row, when odd (whole quads): the request's last takes
    // 0 on the right, any other goes to the halo
    if ((Lb & 3) == 0) {
      const int64_t jl = j0 + Lb - 1;
      if (jl == P.N - 1)
        fz.put(jl, fz.mp + fz.a * (fz.yl + 0.f) + fz.qp * fz.st);
      else {
        const size_t h = (size_t)b * kC + c;
        P.hm[h] = fz.mp;
        P.hq[h] = fz.qp;
        P.hl[h] = fz.yl;
      }
    }
  }
  const bool lane_bad = lane_ok && x != kL;
  if (__ballot(lane_bad) != 0ull || ptr != W) {
    if (lane == 0) set_status(P.status, DCKV_ECORRUPT);
  }
}

// The odd row that ends each block but the last, after the fused decode:
// mu + a (yhat_{j-1} + yhat_{j+1}) + q step from the halo (the same
// expression as the rows decoded in place).  Thread (block b, component c).
__global__ __launch_bounds__(256) void k_dequant_fix(const Batch<DecP> B) {
  const int ri = batch_req(B, blockIdx.x);
  const DecP &P = B.r[ri];
  if (*P.status != 0) return;
  const int64_t i = (int64_t)(blockIdx.x - B.start[ri]) * blockDim.x + threadIdx.x;
  if (i >= (P.n_blk - 1) * (int64_t)kC) return;
  const int64_t b = i / kC;
  const int c = (int)(i - b * kC);
  const size_t h = (size_t)b * kC + c;
  const float st = P.step[c], a = P.nbr[c];
  const float y = P.hm[h] + a * (P.hl[h] + P.hr[h + kC]) + P.hq[h] * st;
  P.yhat_b[(size_t)(kBlock * b + kBlock - 1) * kC + c] = __builtin_bit_cast(uint16_t, (__bf16)y);
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
void launch_rans_encode(const EncodeArgs *args, int n) {
  auto fill = [&](int i) {
    const EncodeArgs &a = args[i];
    EncP P;
    P.tab = a.p->dev.tab;
    P.rcp = a.p->dev.rcp;
    P.sym32 = reinterpret_cast<const uint32_t *>(a.ws + a.l.sym);
    P.scratch = reinterpret_cast<uint16_t *>(a.ws + a.l.scratch);
    P.gwords = reinterpret_cast<uint32_t *>(a.ws + a.l.gwords);
    P.N = a.g.N;
    P.N256 = a.g.N256;
    P.n_blk = a.g.n_blk;
    P.Ca = a.p->C_a;
    P.G = a.p->G;
    P.status = a.status;
    return P;
  };
  auto count = [&](int i) {
    const EncodeArgs &a = args[i];
    return a.g.n_groups == 0 ? 0u : (uint32_t)(((a.g.n_blk + kEncWaves - 1) / kEncWaves) * a.p->G);
  };
  launch_batched<EncP>(k_rans_encode, "rans_encode", n, args[0].s, kEncWaves * 64, fill, count);
}

void launch_scan_header(const EncodeArgs *args, int n) {
  auto fill = [&](int i) {
    const EncodeArgs &a = args[i];
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
    return P;
  };
  launch_batched<ScanP>(k_scan_header, "scan", n, args[0].s, 1024, fill, [](int) { return 1u; });
}

void launch_pack(const EncodeArgs *args, int n) {
  auto fill = [&](int i) {
    const EncodeArgs &a = args[i];
    PackP P;
    P.scratch = reinterpret_cast<const uint16_t *>(a.ws + a.l.scratch);
    P.gwords = reinterpret_cast<const uint32_t *>(a.ws + a.l.gwords);
    P.goffs = reinterpret_cast<const uint64_t *>(a.ws + a.l.goffs);
    P.esc_sorted = reinterpret_cast<const uint32_t *>(a.ws + a.l.esc_sorted);
    P.ws = a.ws;
    P.stream = a.stream;
    P.n_groups = a.g.n_groups;
    P.status = a.status;
    return P;
  };
  // one workgroup per group, at most 4,096 per request (at least one, for the
  // escape records)
  auto count = [&](int i) { return (uint32_t)std::max<int64_t>(1, args[i].g.n_groups); };
  launch_batched<PackP>(k_pack, "pack", n, args[0].s, 256, fill, count);
}

void launch_parse(const DecodeArgs *args, int n, bool with_rope) {
  auto rope_blocks = [&](int i) {
    const int64_t n_rope = with_rope ? (256 + args[i].g.rope_hi) * kHalf : 0;
    return (uint32_t)std::min<int64_t>((n_rope + 255) / 256, 4096);
  };
  auto fill = [&](int i) {
    const DecodeArgs &a = args[i];
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
    return P;
  };
  launch_batched<ParseP>(k_parse, "parse", n, args[0].s, 256, fill, [&](int i) { return 1u + rope_blocks(i); });
}

void launch_rans_decode(const DecodeArgs *args, int n) {
  auto fill = [&](int i) {
    const DecodeArgs &a = args[i];
    DecP P{};
    P.tab = a.p->dev.tab;
    P.bucket = a.p->dev.bucket;
    P.fuse = dequant_fused(a) ? 1 : 0;
    P.mtab = a.p->mtab;
    P.tok = a.tok;
    P.step = a.p->dev.step;
    P.nbr = a.p->dev.nbr;
    P.yhat_b = reinterpret_cast<uint16_t *>(a.ws + a.l.yhat_b);
    P.hm = reinterpret_cast<float *>(a.ws + a.l.halo_a);
    P.hq = reinterpret_cast<float *>(a.ws + a.l.halo_b);
    P.hl = reinterpret_cast<float *>(a.ws + a.l.dhalo);
    P.hr = reinterpret_cast<float *>(a.ws + a.l.dhalo) + (size_t)a.g.n_mtiles * a.p->C;
    P.keep_head = a.p->keep_head;
    P.vocab = a.p->vocab;
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
    return P;
  };
  auto count = [&](int i) {
    const DecodeArgs &a = args[i];
    return a.g.n_groups == 0 ? 0u : (uint32_t)(((a.g.n_blk + kDecWaves - 1) / kDecWaves) * a.p->G);
  };
  launch_batched<DecP>(k_rans_decode, "rans_decode", n, args[0].s, kDecWaves * 64, fill, count);
  // the odd rows that end the blocks of the fused requests
  auto fix_count = [&](int i) {
    const DecodeArgs &a = args[i];
    if (!dequant_fused(a) || a.g.n_blk < 2) return 0u;
    return (uint32_t)(((a.g.n_blk - 1) * (int64_t)a.p->C + 255) / 256);
  };
  launch_batched<DecP>(k_dequant_fix, "dequant_fix", n, args[0].s, 256, fill, fix_count);
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
