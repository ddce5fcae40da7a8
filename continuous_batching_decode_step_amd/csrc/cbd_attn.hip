// Ragged per-lane grouped-query attention for one decode step on gfx950.
//
// "MODEL-BATCHING-RESULTS — multi-user batched decode, measured" (section
// "The lever") keeps attention per user: lane b's queries read only lane b's
// own cache, over its own length.  A lane's cache is a list of blocks of a
// shared pool, one per 64-position chunk; within a block one (layer, KV head)
// chunk is a contiguous run, and a work item names the blocks of its chunks.
// There is no padding across lanes: a lane at position p reads slots [0, p]
// (the tail of its last chunk is masked) and writes slot p.
//
// Two kernels produce per-chunk partials.  The matrix-core kernel (bf16 KV,
// head_dim 64/128, k_attn_mf) takes one workgroup per (lane, KV head, aligned
// group of ATTN_GROUP chunks of ATTN_SPLIT = 64 keys), one wave per chunk,
// and merges the group's chunks in LDS into one partial.  The general kernel
// (k_attn) takes one workgroup of one wave per (lane, KV head, chunk), or, in
// launches with few such waves, per (lane, query head, chunk), so a single
// lane's keys spread over many CUs.  Inside the general kernel's wave, 16
// lanes share one key row: lane
// (r, c) = (lane / 16, lane % 16) holds dims [c*D, c*D + D) of key 4*it + r
// for it = 0..15, D = hd / 16, so every load instruction reads 4 whole rows
// (coalesced 16-byte loads for hd = 128 bf16 and hd = 64 f32).  A whole-group
// wave scores the group's query heads (all heads sharing the KV head)
// together, so each K and V row is read once per group.  Scores are f32 dot products of the
// rotated f32 query with the stored keys; a reduce-scatter across the 16
// lanes of a row leaves lane (r, c) with the score of key 4c + r.  Softmax
// statistics and the value sum are exact f32 per chunk; partials meet in a
// second, small kernel that rescales by each partial's max and sums them in
// order.  Chunk and group sizes are constants, so a lane's result depends on
// its own position only, never on B or on other lanes.
//
// The workgroup whose chunk holds slot p rotates the new key at p (the same
// position as the queries: "parallel-slots.md", "S1b decode: design traps",
// trap 2), rounds K and V to the KV format, writes them in place, and uses
// the rounded values for key p.
#include <algorithm>
#include <type_traits>

#include "cbd_internal.h"

namespace cbd {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline uint16_t f2bf_a(float f) {
  unsigned u = __builtin_bit_cast(unsigned, f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ inline float bf2f(unsigned h16) { return __builtin_bit_cast(float, h16 << 16); }

// One attention output in the activation format act (WT_F32, WT_BF16, WT_Q8).
__device__ inline void put_out(void* base, size_t idx, float v, int act) {
  if (act == WT_F32)
    ((float*)base)[idx] = v;
  else if (act == WT_BF16)
    ((uint16_t*)base)[idx] = f2bf_a(v);
  else
    ((_Float16*)base)[idx] = (_Float16)v;
}

// D consecutive KV elements (D = hd/16) of one key as loaded (raw words), and
// their f32 values.  Loading and converting are separate so that a whole
// batch of loads can be issued before the first one is waited for.
template <int D, bool BF>
struct KVRaw {
  static constexpr int BYTES = D * (BF ? 2 : 4);
  static constexpr int NW = BYTES >= 4 ? BYTES / 4 : 1;
  unsigned w[NW];
};

template <int D, bool BF>
__device__ inline KVRaw<D, BF> load_raw(const void* base, long long off) {
  KVRaw<D, BF> r;
  constexpr int BYTES = KVRaw<D, BF>::BYTES;
  const char* p = (const char*)base + off * (BF ? 2 : 4);
  if constexpr (BYTES >= 16) {
#pragma unroll
    for (int h = 0; h < BYTES / 16; ++h) {
      const u32x4 v = *((const u32x4*)p + h);
      r.w[4 * h] = v.x;
      r.w[4 * h + 1] = v.y;
      r.w[4 * h + 2] = v.z;
      r.w[4 * h + 3] = v.w;
    }
  } else if constexpr (BYTES == 8) {
    const u32x2 v = *(const u32x2*)p;
    r.w[0] = v.x;
    r.w[1] = v.y;
  } else if constexpr (BYTES == 4) {
    r.w[0] = *(const unsigned*)p;
  } else {
    r.w[0] = *(const uint16_t*)p;
  }
  return r;
}

// x := (x & keep) | (n & take), word by word: keeps the loaded key, or puts
// the new one in its place, or zeroes it, without branches.
template <int D, bool BF>
__device__ inline void raw_select(KVRaw<D, BF>& x, unsigned keep, unsigned take, const KVRaw<D, BF>& n) {
#pragma unroll
  for (int i = 0; i < KVRaw<D, BF>::NW; ++i) x.w[i] = (x.w[i] & keep) | (n.w[i] & take);
}

template <int D, bool BF>
__device__ inline void raw_to_f32(const KVRaw<D, BF>& r, float (&v)[D]) {
  if constexpr (BF) {
    if constexpr (D == 1) {
      v[0] = __builtin_bit_cast(float, r.w[0] << 16);
    } else {
#pragma unroll
      for (int e = 0; e < D / 2; ++e) {
        v[2 * e] = __builtin_bit_cast(float, r.w[e] << 16);
        v[2 * e + 1] = __builtin_bit_cast(float, r.w[e] & 0xffff0000u);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < D; ++e) v[e] = __builtin_bit_cast(float, r.w[e]);
  }
}

// Rotate-half RoPE of one element: x is dim d of a head vector, y its
// partner (dim d + hd/2 for the first half, d - hd/2 for the second), t the
// pair's (cos, sin).  Every kernel that rotates a key or a query calls this one
// expression, so a key appended by one kernel equals the key another uses.
__device__ inline float rope_pair(float x, float y, float2 t, bool first) {
  return first ? x * t.x - y * t.y : x * t.x + y * t.y;
}

// G: query heads per wave, a divisor of the group size a.G; the a.G / G waves
// of one (item, KV head) are numbered 8 apart, so they land on one XCD and
// share the chunk's loads in its L2.
template <int HD, bool KVBF16, int G>
__global__ __launch_bounds__(64) void k_attn(AttnArgs a) {
  constexpr int D = HD / 16;  // dims per lane
  static_assert(ATTN_SPLIT == 64, "one wave holds 4 keys x 16 iterations");
  const int nz = a.G / G;  // waves per (item, KV head)
  const int zb = blockIdx.x >> 3;
  const int item = (zb / nz) * 8 + (blockIdx.x & 7);
  const int jz = (zb % nz) * G;  // this wave's first head of the group
  const int g = blockIdx.y;
  const int lane = threadIdx.x;
  const int r = lane >> 4, c = lane & 15;
  // The item and the step's item count in one memory round trip, and the
  // item carries the row's position, so the key loads wait on nothing else.
  // The grid is sized for the most items a step can have: an item past the
  // count reads lane 0's chunk 0 (in bounds, never used) and leaves before
  // it writes anything.
  const int n_items = *a.n_items_dev;
  const int il = min(item, a.max_items - 1);  // the grid rounds items up to 8
  int4 it4r = *(const int4*)(a.items + ITEM_INTS * il);
  int blkr = a.items[ITEM_INTS * il + 4];  // the chunk's block
  // an opaque use of the item here keeps its loads beside the count's (the
  // compiler would otherwise load it only after testing the count)
  __asm__ volatile("" : "+s"(it4r.x), "+s"(it4r.y), "+s"(it4r.z), "+s"(blkr));
  const bool valid = item < n_items;
  const int blk = valid ? blkr : 0;
  const int b = valid ? (it4r.x & 0xffffff) : 0;
  const int s = valid ? it4r.y : 0;  // one chunk per item for this kernel
  const int p = valid ? it4r.z : 0;
  const int nk = p + 1;
  const int kbeg = s * ATTN_SPLIT;  // first key of the chunk
  const int kend = min(kbeg + ATTN_SPLIT, nk);

  // key t of the chunk sits at base + t * HD (base is the chunk's block, minus kbeg keys)
  const long long base = (long long)blk * a.block_elems + a.layer_off + (long long)g * ATTN_SPLIT * HD -
                         (long long)kbeg * HD;
  const float* row = a.qkv + (size_t)b * a.Nqkv;
  const float2* cs = a.rope + (size_t)b * (HD / 2);
  const int d0 = c * D;  // first dim of this lane
  // rotation partner of dim d is d + hd/2 (first half) or d - hd/2 (second half)
  const bool first_half = d0 < HD / 2;
  const int dp = first_half ? d0 + HD / 2 : d0 - HD / 2;

  // Batches of KB keys (and values) are loaded before any is used
  // (unconditional, from a key clamped into range; key p and keys past the
  // end are replaced after the load, since slot p may be being written).  A
  // one-head wave (a launch with few waves, bound by its serial chain) issues
  // the first batch of keys and of values before anything waits on memory; a
  // whole group's wave issues its keys after its queries and its values after
  // its scores, as their registers would otherwise cut its occupancy (100 ->
  // 192 VGPRs for three heads of 64 dims: 10-15% slower per step at 256-960
  // lanes).
  constexpr int KB = KVRaw<D, KVBF16>::BYTES > 16 ? 8 : 16;
  constexpr bool EARLY = G == 1;
  KVRaw<D, KVBF16> kr0[KB], vr[KB];
  auto load_k0 = [&]() {
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const int key = kbeg + 4 * i + r;
      kr0[i] = load_raw<D, KVBF16>(a.kpool, base + (long long)min(key, kend - 1) * HD + d0);
    }
  };
  auto load_v0 = [&]() {
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const int key = kbeg + 4 * i + r;
      vr[i] = load_raw<D, KVBF16>(a.vpool, base + (long long)min(key, kend - 1) * HD + d0);
    }
  };
  if constexpr (EARLY) {
    load_k0();
    load_v0();
  }
  if (!valid) return;

  // Rotated queries of the group for this lane's dims (f32).
  float q[G][D];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float* qh = row + (size_t)(g * a.G + jz + j) * HD;
#pragma unroll
    for (int e = 0; e < D; ++e) {
      const int jj = first_half ? d0 + e : d0 + e - HD / 2;
      const float2 t = cs[jj];
      q[j][e] = rope_pair(qh[d0 + e], qh[dp + e], t, first_half);
    }
  }
  // The new key and value at slot p, rotated and rounded to the KV format
  // (kept as stored words).
  // Fused mode: the item whose chunk holds slot p rotates and writes the new
  // key and value and uses them for that slot.  Attend-only mode reads slot p
  // from the cache like any key (k_kv_append wrote it).
  const bool fused = a.mode == ATTN_FUSED;
  const bool has_new = fused && nk > s * ATTN_SPLIT && nk <= s * ATTN_SPLIT + ATTN_SPLIT;
  const int pk = fused ? p : nk;  // keys below pk are read from the cache
  KVRaw<D, KVBF16> knr, vnr;
#pragma unroll
  for (int i = 0; i < KVRaw<D, KVBF16>::NW; ++i) knr.w[i] = vnr.w[i] = 0u;
  if (has_new) {
    const float* kr = row + (size_t)(a.Hq + g) * HD;
    const float* vr = row + (size_t)(a.Hq + a.Hkv + g) * HD;
    float kn[D], vn[D];
#pragma unroll
    for (int e = 0; e < D; ++e) {
      const int jj = first_half ? d0 + e : d0 + e - HD / 2;
      const float2 t = cs[jj];
      kn[e] = rope_pair(kr[d0 + e], kr[dp + e], t, first_half);
      vn[e] = vr[d0 + e];
    }
    if constexpr (KVBF16) {
      if constexpr (D == 1) {
        knr.w[0] = f2bf_a(kn[0]);
        vnr.w[0] = f2bf_a(vn[0]);
      } else {
#pragma unroll
        for (int e = 0; e < D / 2; ++e) {
          knr.w[e] = (unsigned)f2bf_a(kn[2 * e]) | ((unsigned)f2bf_a(kn[2 * e + 1]) << 16);
          vnr.w[e] = (unsigned)f2bf_a(vn[2 * e]) | ((unsigned)f2bf_a(vn[2 * e + 1]) << 16);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < D; ++e) {
        knr.w[e] = __builtin_bit_cast(unsigned, kn[e]);
        vnr.w[e] = __builtin_bit_cast(unsigned, vn[e]);
      }
    }
    if (r == 0 && jz == 0) {  // one row of lanes of the group's first wave writes the slot
      const long long o = base + (long long)p * HD + d0;
#pragma unroll
      for (int e = 0; e < D; ++e) {
        if constexpr (KVBF16) {
          const unsigned kw = D == 1 ? knr.w[0] : knr.w[e / 2] >> (16 * (e & 1));
          const unsigned vw = D == 1 ? vnr.w[0] : vnr.w[e / 2] >> (16 * (e & 1));
          ((uint16_t*)a.kpool)[o + e] = (uint16_t)kw;
          ((uint16_t*)a.vpool)[o + e] = (uint16_t)vw;
        } else {
          ((unsigned*)a.kpool)[o + e] = knr.w[e];
          ((unsigned*)a.vpool)[o + e] = vnr.w[e];
        }
      }
    }
  }

  // Scores of the wave's 64 keys: lane (r, c) accumulates its D dims of key
  // kbeg + 4*it + r into part[it][j]; the row then reduce-scatters so that
  // lane (r, c) ends with the full score of key kbeg + 4*c + r.  Loads are
  // issued in batches of KB keys before any is used (the first batch above).
  if constexpr (!EARLY) load_k0();
  const float inv = 1.0f / sqrtf((float)HD);
  // Keys of the chunk up to the row's end.  One-head waves skip groups of 16
  // keys past it below: their probabilities are exactly 0 and their values
  // 0, so their terms (+0) change no sum.  (In a whole group's wave the
  // branches leave the compiler short of scalar registers: ~1000 spills to
  // vector lanes, 25.5 -> 39.1 us per launch at 960 lanes.)
  const int nlive = kend - kbeg;
  float part[16][G];
#pragma unroll
  for (int i0 = 0; i0 < 16; i0 += KB) {
    KVRaw<D, KVBF16> kr[KB];
    if (i0 == 0) {
#pragma unroll
      for (int i = 0; i < KB; ++i) kr[i] = kr0[i];
    } else {
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        const int key = kbeg + 4 * (i0 + i) + r;
        kr[i] = load_raw<D, KVBF16>(a.kpool, base + (long long)min(key, kend - 1) * HD + d0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      if (EARLY && 4 * ((i0 + i) & ~3) >= nlive) {  // 16 keys all past the end: their scores are masked
#pragma unroll
        for (int j = 0; j < G; ++j) part[i0 + i][j] = 0.f;
        continue;
      }
      const int key = kbeg + 4 * (i0 + i) + r;
      const unsigned take = fused && key == p ? ~0u : 0u;
      const unsigned keep = key < pk ? ~0u : 0u;  // past the end: zero
      raw_select<D, KVBF16>(kr[i], keep, take, knr);
      float kv[D];
      raw_to_f32<D, KVBF16>(kr[i], kv);
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) acc += q[j][e] * kv[e];
        part[i0 + i][j] = acc;
      }
    }
  }
  if constexpr (!EARLY) {
    load_v0();  // in flight during the softmax
    __builtin_amdgcn_sched_barrier(0);
  }
  float sc[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float v[16];
#pragma unroll
    for (int it = 0; it < 16; ++it) v[it] = part[it][j];
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) {
      const bool upper = (c & m) != 0;
#pragma unroll
      for (int i = 0; i < m; ++i) {
        const float send = upper ? v[i] : v[i + m];
        const float keep = upper ? v[i + m] : v[i];
        v[i] = keep + __shfl_xor(send, m);
      }
    }
    const int key = kbeg + 4 * c + r;
    sc[j] = key < kend ? v[0] * inv : -INFINITY;
  }

  // Softmax statistics over the chunk's 64 keys.
  float mx[G], pe[G], ls[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float m = sc[j];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
    mx[j] = m;
    pe[j] = sc[j] == -INFINITY ? 0.f : expf(sc[j] - m);
    float l = pe[j];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) l += __shfl_xor(l, off);
    ls[j] = l;
  }

  // Values: lane (r, c) accumulates p * V over keys kbeg + 4*it + r for its dims.
  float o[G][D];
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int e = 0; e < D; ++e) o[j][e] = 0.f;
#pragma unroll
  for (int i0 = 0; i0 < 16; i0 += KB) {
    if (i0 > 0) {
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        const int key = kbeg + 4 * (i0 + i) + r;
        vr[i] = load_raw<D, KVBF16>(a.vpool, base + (long long)min(key, kend - 1) * HD + d0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const int it = i0 + i;
      if (EARLY && 4 * (it & ~3) >= nlive) continue;
      const int key = kbeg + 4 * it + r;
      const unsigned take = fused && key == p ? ~0u : 0u;
      const unsigned keep = key < pk ? ~0u : 0u;
      raw_select<D, KVBF16>(vr[i], keep, take, vnr);
      float vv[D];
      raw_to_f32<D, KVBF16>(vr[i], vv);
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float pj = __shfl(pe[j], r * 16 + it);  // the probability of key 4*it + r
#pragma unroll
        for (int e = 0; e < D; ++e) o[j][e] += pj * vv[e];
      }
    }
  }
  // Sum the four rows (fixed butterfly) and publish the chunk's (o, m, l) for
  // the combine kernel.
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int e = 0; e < D; ++e) {
      float v = o[j][e];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      o[j][e] = v;
    }
  if (nk <= ATTN_SPLIT) {  // the row's only partial: the combine's o / l (the combine skips the row)
    if (r == 0) {
#pragma unroll
      for (int j = 0; j < G; ++j)
#pragma unroll
        for (int e = 0; e < D; ++e)
          put_out(a.out, (size_t)b * a.Hq * HD + (size_t)(g * a.G + jz + j) * HD + d0 + e, o[j][e] / ls[j], a.act);
    }
    return;
  }
  const size_t pstride = (size_t)a.G * (HD + 2);
  float* dst = a.part + (((size_t)b * a.max_splits + s) * a.Hkv + g) * pstride + (size_t)jz * (HD + 2);
  if (r == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < D; ++e) dst[(size_t)j * (HD + 2) + d0 + e] = o[j][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      dst[(size_t)j * (HD + 2) + HD] = mx[j];
      dst[(size_t)j * (HD + 2) + HD + 1] = ls[j];
    }
  }
}


// ---- bf16 KV: scores and P.V on the matrix cores ---------------------------------
//
// Same work and the same per-chunk results contract as k_attn (chunk partials
// (o, m, l) of 64 keys, combined in chunk order by k_attn_combine), with both
// products on MFMA (v_mfma_f32_16x16x32_bf16).
//
// Scores: for each 16-key tile, S^T[key][col] over head_dim with the keys (bf16,
// as stored) as the A operand and, as the B operand, each query head's rotated
// f32 query split into bf16 parts, q = hi + mid + lo exactly (hi = bf16(q),
// mid = bf16(q - hi), lo = q - hi - mid, which has at most 8 significant bits),
// in columns CPH*j, CPH*j + 1 and CPH*j + 2 of head j; the score is hi + (mid +
// lo).  Products of bf16 values are exact in f32, so each score is the f32 sum
// of the exact products.  With more than four query heads per KV head (CPH = 2)
// the lo part is dropped (q = hi + mid + O(2^-18 |q|)).
//
// P.V: the probabilities p (f32) split the same way into bf16 parts, in the A
// operand's rows CPH*j + part, against the values as the B operand; head j's
// output is the f32 sum hi + (mid + lo) of its part rows.  Since p = hi + mid +
// lo exactly, every product is exact and the sums are f32 sums of the exact
// products, as the f32 vector path gives.
//
// Lane roles (l16 = lane % 16, g4 = lane / 16): the score tile leaves S[key
// 16t + 4*g4 + i][col l16] in lane (l16, g4), register (t, i); the four lanes
// of head j's columns combine its parts by quad-lane DPP and so all hold its
// score, softmax statistics and p for those keys.  The P.V A operand of lane
// (row l16, g4) over a 32-key block u is exactly those 8 keys (k = 8*g4 + e for
// key 32u + 16*(e >> 2) + 4*g4 + (e & 3)), so the lane forms its part of p in
// registers, and the values are stored in that key order (vfrag_off): one
// 16-byte load per (dim tile, key block).
__device__ inline u32x4 zero4a() { return u32x4{0u, 0u, 0u, 0u}; }

// Buffer-descriptor loads over one chunk of one (layer, KV head) in its block:
// a byte offset at or past the descriptor's range reads zeros without
// touching memory (the raw buffer range check), which lets a wave without a
// chunk be switched off by its offset alone.  Descriptor word 3 = 0x00020000
// (32-bit data format) on gfx9 parts.
constexpr unsigned PAST_RANGE = 0x80000000u;  // an offset past any chunk's range

__device__ inline __amdgpu_buffer_rsrc_t chunk_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ inline u32x4 chunk_ld16(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// Quad-lane DPP broadcast: every lane takes lane Q of its group of four (a
// vector-ALU operand modifier, no trip through the LDS crossbar).
template <int CTRL>
__device__ inline float quad_perm(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v),
                                                               CTRL, 0xF, 0xF, false));
}

// Score columns per query head and bf16 parts of each query and probability.
template <int G>
struct MfCols {
  static constexpr int CPH = G <= 4 ? 4 : 2;
  static constexpr int NQ = CPH == 4 ? 3 : 2;
  static_assert(G >= 1 && G * CPH <= 16, "query heads per KV head");
};

// Two f32 values to packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ inline unsigned pk_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(unsigned, v);
}

// Part `part` (0 hi, 1 mid, 2 lo, else zero) of two probabilities, packed:
// hi = bf16(p), mid = bf16(p - hi), lo = bf16(p - hi - mid); each difference
// is exact, so hi + mid + lo = p exactly.
__device__ inline unsigned p_part2(float a, float b, int part) {
  const unsigned hi = pk_bf16(a, b);
  const float ra = a - __builtin_bit_cast(float, hi << 16), rb = b - __builtin_bit_cast(float, hi & 0xffff0000u);
  const unsigned mid = pk_bf16(ra, rb);
  const float sa = ra - __builtin_bit_cast(float, mid << 16), sb = rb - __builtin_bit_cast(float, mid & 0xffff0000u);
  const unsigned lo = pk_bf16(sa, sb);
  return part == 0 ? hi : part == 1 ? mid : part == 2 ? lo : 0u;
}

// The per-chunk work of a wave, shared by the decode kernel (k_attn_mf) and
// the prefill kernel (k_attn_rows) so that both give the same bits.
//
// Scores of one 64-key chunk: four 16-key tiles, each a chain of MFMAs over
// head_dim with the keys as the A operand (kr[t][kk]: fragment (t, kk) of the
// chunk) and the query parts as the B operand.
template <int HD>
__device__ inline void mf_scores(const u32x4 (&kr)[4][HD / 32], const u32x4 (&bq)[HD / 32], f32x4 (&sc)[4]) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < HD / 32; ++kk)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[t][kk]),
                                                    __builtin_bit_cast(bf16x8, bq[kk]), acc, 0, 0, 0);
    sc[t] = acc;
  }
}

// Value fragments vf[u][dt] of a chunk with the keys at or past pk zeroed and,
// if has_new, key p (in this chunk) replaced by the new value vn (bf16 words,
// dims 0..HD-1, in LDS).  kb: the chunk's first key.
template <int HD>
__device__ inline void mf_mask_v(u32x4 (&vf)[2][HD / 16], int kb, int pk, bool has_new, int p, int g4, int l16,
                                 const uint16_t* vn) {
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // dword w holds keys e = 2w, 2w + 1: key 32u + 16*(w >> 1) + 4*g4 + 2*(w & 1) (+1)
      const int k0 = kb + 32 * u + 16 * (w >> 1) + 4 * g4 + 2 * (w & 1);
      const unsigned keep = (k0 < pk ? 0xffffu : 0u) | (k0 + 1 < pk ? 0xffff0000u : 0u);
      const unsigned take = !has_new ? 0u : k0 == p ? 0xffffu : k0 + 1 == p ? 0xffff0000u : 0u;
#pragma unroll
      for (int dt = 0; dt < HD / 16; ++dt) {
        unsigned x = vf[u][dt][w] & keep;
        if (take) {
          const unsigned nv = vn[16 * dt + l16];
          x = (x & ~take) | ((nv | (nv << 16)) & take);
        }
        vf[u][dt][w] = x;
      }
    }
}

// Softmax statistics and P.V of the chunk from its scores and its value
// fragments (masked): keys below ke count.  Leaves, in lane (l16, g4), the
// output o[r][dt] = dim 16*dt + l16 of the head of part row 4*g4 + r*CPH (r <
// 4 / CPH; CPH = 4: head g4, CPH = 2: heads 2*g4 and 2*g4 + 1), and head
// l16 / CPH's maximum m and sum l (every lane).
template <int HD, int G>
__device__ inline void mf_softmax_pv(const f32x4 (&sc)[4], const u32x4 (&vf)[2][HD / 16], int kb, int ke, int g4,
                                     int l16, float (&o)[4 / MfCols<G>::CPH][HD / 16], float& m, float& l) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  constexpr int CPH = MfCols<G>::CPH;
  constexpr int DT = HD / 16;
  const float inv = 1.0f / sqrtf((float)HD);
  // hi + (mid + lo) of the lane's head, scale, mask
  float pr[4][4];
  m = -INFINITY;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float s;
      if constexpr (CPH == 4)
        s = quad_perm<0x00>(sc[t][i]) + (quad_perm<0x55>(sc[t][i]) + quad_perm<0xAA>(sc[t][i]));
      else
        s = quad_perm<0xA0>(sc[t][i]) + quad_perm<0xF5>(sc[t][i]);
      const int key = kb + 16 * t + 4 * g4 + i;
      const float v = s * inv;
      pr[t][i] = key < ke ? v : -INFINITY;
      m = fmaxf(m, pr[t][i]);
    }
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  // exponentials by the hardware exp2 with the log2(e) scale (about 1 ulp;
  // this path serves bf16 caches only)
  l = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[t][i] = pr[t][i] == -INFINITY ? 0.f : __expf(pr[t][i] - m);
      l += pr[t][i];
    }
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);

  // A operand of key block u: this lane's part of p for keys 32u + 16*(e >> 2) + 4*g4 + (e & 3)
  const int part = l16 % CPH;
  u32x4 pa[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int t = 2 * u + (w >> 1), i = 2 * (w & 1);
      pa[u][w] = p_part2(pr[t][i], pr[t][i + 1], part);
    }
  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 2; ++u)
      a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pa[u]), __builtin_bit_cast(bf16x8, vf[u][dt]),
                                                  a, 0, 0, 0);
    acc[dt] = a;
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    if constexpr (CPH == 4) {
      o[0][dt] = acc[dt][0] + (acc[dt][1] + acc[dt][2]);
    } else {
      o[0][dt] = acc[dt][0] + acc[dt][1];
      o[1][dt] = acc[dt][2] + acc[dt][3];
    }
  }
}

// A group's chunk partials merged in chunk order into one partial: with
// M = max(Mr, m_k), Lr = Lr e^(Mr - M) + l_k e^(m_k - M), likewise Or
// (starting from Mr = -inf, Lr = Or = 0, so one chunk gives exactly its own
// o and l).  ms/ls: chunk k's statistics at [k * st]; os: its output at [k * ost].
struct Merged {
  float o, l, m;
};
__device__ inline Merged merge_chunks(int nc, const float* ms, const float* ls, int st, const float* os, int ost) {
  float Mr = -INFINITY, Lr = 0.f, Or = 0.f;
  for (int k = 0; k < nc; ++k) {
    const float mk = ms[k * st];
    const float M = fmaxf(Mr, mk);
    const float sa = __expf(Mr - M), sb = __expf(mk - M);
    Lr = __builtin_fmaf(Lr, sa, ls[k * st] * sb);
    Or = __builtin_fmaf(Or, sa, os[k * ost] * sb);
    Mr = M;
  }
  return Merged{Or, Lr, Mr};
}

// Rotated query parts of the group's G heads (f32 head vectors at qv + j*HD,
// rotation table cs) into the score B-operand rows qs[CPH*j + part], in two
// stages so that a caller can load one row's inputs while it stores another's:
// element idx = j*HD + d takes dim d of head j and its rotation partner.
struct QIn {
  float x, y;
  float2 t;
};
template <int HD>
__device__ inline QIn mf_query_in(const float* qv, const float2* cs, int idx) {
  const int j = idx / HD, d = idx % HD;
  const bool fh = d < HD / 2;
  const float* v = qv + (size_t)j * HD;
  return QIn{v[d], v[fh ? d + HD / 2 : d - HD / 2], cs[fh ? d : d - HD / 2]};
}
template <int HD, int G>
__device__ inline void mf_query_out(const QIn& in, int idx, uint16_t (*qs)[HD]) {
  constexpr int CPH = MfCols<G>::CPH;
  const int j = idx / HD, d = idx % HD;
  const float q = rope_pair(in.x, in.y, in.t, d < HD / 2);
  const uint16_t hi = f2bf_a(q);
  const float r1 = q - bf2f(hi);  // exact
  const uint16_t mid = f2bf_a(r1);
  qs[CPH * j][d] = hi;
  qs[CPH * j + 1][d] = mid;
  if constexpr (MfCols<G>::NQ == 3) qs[CPH * j + 2][d] = f2bf_a(r1 - bf2f(mid));  // exact: at most 8 significant bits
}
template <int HD, int G>
__device__ inline void mf_prep_queries(const float* qv, const float2* cs, uint16_t (*qs)[HD], int tid, int nthr) {
  for (int idx = tid; idx < G * HD; idx += nthr) mf_query_out<HD, G>(mf_query_in<HD>(qv, cs, idx), idx, qs);
}

// The score B operand of lane (col l16, g4) from the query rows in LDS (zero
// for the columns no part uses).
template <int HD, int G>
__device__ inline void mf_load_bq(const uint16_t (*qs)[HD], int l16, int g4, u32x4 (&bq)[HD / 32]) {
  constexpr int CPH = MfCols<G>::CPH;
  const bool used = l16 < CPH * G && l16 % CPH < MfCols<G>::NQ;
#pragma unroll
  for (int kk = 0; kk < HD / 32; ++kk) {
    const u32x4 v = *(const u32x4*)&qs[used ? l16 : 0][kk * 32 + g4 * 8];
    bq[kk] = used ? v : zero4a();
  }
}

// Chunk fragments of one wave: K (score A operand) and V (P.V B operand), one
// 16-byte load per fragment and lane; 1 KB per wave-wide load.
template <int HD>
__device__ inline void mf_load_k(__amdgpu_buffer_rsrc_t krs, unsigned off, u32x4 (&kr)[4][HD / 32]) {
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int kk = 0; kk < HD / 32; ++kk) kr[t][kk] = chunk_ld16(krs, off + (t * (HD / 32) + kk) * 1024);
}
template <int HD>
__device__ inline void mf_load_v(__amdgpu_buffer_rsrc_t vrs, unsigned off, u32x4 (&vf)[2][HD / 16]) {
#pragma unroll
  for (int dt = 0; dt < HD / 16; ++dt)
#pragma unroll
    for (int u = 0; u < 2; ++u) vf[u][dt] = chunk_ld16(vrs, off + (dt * 2 + u) * 1024);
}

// One wave's chunk partial to LDS: outputs of its heads, and the statistics
// (lane l16 = CPH*j of lane row 0 holds head j's).
template <int HD, int G>
__device__ inline void mf_store_partial(const float (&o)[4 / MfCols<G>::CPH][HD / 16], float m, float l, int g4,
                                        int l16, float (*os)[HD], float* ms, float* ls) {
  constexpr int CPH = MfCols<G>::CPH;
#pragma unroll
  for (int r = 0; r < 4 / CPH; ++r) {
    const int j = (4 / CPH) * g4 + r;
    if (j < G) {
#pragma unroll
      for (int dt = 0; dt < HD / 16; ++dt) os[j][16 * dt + l16] = o[r][dt];
    }
  }
  if (g4 == 0 && l16 % CPH == 0 && l16 / CPH < G) {
    ms[l16 / CPH] = m;
    ls[l16 / CPH] = l;
  }
}

// One workgroup per (lane, KV head, aligned group of ATTN_GROUP chunks), one
// wave per chunk.  Each wave computes its chunk's partial (o, m, l) exactly as
// a one-chunk work item would; the partials meet in LDS and are merged in
// chunk order (merge_chunks) into the group's partial.  The group is a
// function of the lane's position only, so the result never depends on B.  A
// row whose keys all fit its first group (its only partial) gets its output
// o / l written here, and the combine skips it.
constexpr int MF_WAVES = ATTN_GROUP;

template <int HD, int G>
__global__ __launch_bounds__(64 * MF_WAVES) __attribute__((amdgpu_waves_per_eu(2))) void k_attn_mf(AttnArgs a) {
  constexpr int KK = HD / 32;   // MFMA k-steps over head_dim
  constexpr int DT = HD / 16;   // 16-dim tiles of the output
  constexpr int CPH = MfCols<G>::CPH;
  static_assert(ATTN_SPLIT == 64, "four 16-key tiles, two 32-key blocks");

  // workgroups in item-major order (the KV heads of one item adjacent), and
  // the items in the order the host lists them: whole groups first, the
  // shorter last groups after them, so the launch drains on the cheapest work
  const int item = blockIdx.x / a.Hkv;
  if (item >= *a.n_items_dev) return;  // the whole workgroup leaves together
  const int g = blockIdx.x % a.Hkv;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int4 it4 = *(const int4*)(a.items + ITEM_INTS * item);
  const int4 bl4 = *(const int4*)(a.items + ITEM_INTS * item + 4);  // blocks of the group's chunks
  const int b = it4.x & 0xffffff, nc = it4.x >> 24, c0 = it4.y, p = it4.z;
  const int nk = p + 1;
  const int c = c0 + w;  // this wave's chunk
  // Fused mode: the lane's last group (its last chunk holds slot p) rotates
  // and writes the new key and value and uses them for that slot.  Attend-only
  // mode: slot p is read from the cache like any key.
  const bool fused = a.mode == ATTN_FUSED;
  const bool holds_p = fused && p / ATTN_SPLIT == c0 + nc - 1;
  const int pk = fused ? p : nk;  // keys below pk are read from the cache
  const bool active = w < nc;     // waves that attend to a chunk
  // (layer, head) offset inside a block; base: this wave's chunk (inactive
  // waves: the last chunk's, never read); pbase: the group's last chunk,
  // which holds slot p when the group is the lane's last
  const long long hoff = a.layer_off + (long long)g * ATTN_SPLIT * HD;
  const int myblk = w == 0 ? bl4.x : w == 1 ? bl4.y : w == 2 ? bl4.z : bl4.w;
  const int lastblk = nc == 1 ? bl4.x : nc == 2 ? bl4.y : nc == 3 ? bl4.z : bl4.w;
  const long long base = (long long)(active ? myblk : lastblk) * a.block_elems + hoff;
  const long long pbase = (long long)lastblk * a.block_elems + hoff;
  const float* row = a.qkv + (size_t)b * a.Nqkv;
  const float2* cs = a.rope + (size_t)b * (HD / 2);
  const uint16_t* kpool = (const uint16_t*)a.kpool;
  const uint16_t* vpool = (const uint16_t*)a.vpool;

  // Whole chunks are read (a block holds whole chunks), and the slots past p
  // (old or never written) are masked or zeroed after the load.  A wave
  // without a chunk loads at an offset past its chunk's buffer: zeros, no access.
  const unsigned chunk_bytes = (unsigned)ATTN_SPLIT * HD * 2;
  const __amdgpu_buffer_rsrc_t krs = chunk_rsrc(kpool + base, chunk_bytes);
  const __amdgpu_buffer_rsrc_t vrs = chunk_rsrc(vpool + base, chunk_bytes);
  const unsigned foff = active ? (unsigned)lane * 16 : PAST_RANGE;
  u32x4 kr[4][KK];
  mf_load_k<HD>(krs, foff, kr);
  // The lane's rotary table goes to LDS now, so its loads overlap the K loads
  // and the query inputs' (the rotation below reads it from there).
  __shared__ float2 css[HD / 2];
  const float2 csv = cs[tid % (HD / 2)];
  // The workgroup rotates the group's queries (split into bf16 parts) and, if
  // its last chunk holds slot p, the new key and value, through LDS; lanes
  // then read their MFMA operand rows from there.
  __shared__ __attribute__((aligned(16))) uint16_t qs[16][HD];
  __shared__ __attribute__((aligned(16))) uint16_t kvn[2][HD];
  __shared__ float os[MF_WAVES][G][HD], ms[MF_WAVES][G], ls[MF_WAVES][G];
  // When the QKV projection ran in split mode without its fold, the workgroup
  // adds the split partials of the values it needs itself, in split order, as
  // the fold would: P_s of lane b at [(s * B + b) * Nqkv + n].  The sums (the
  // group's queries, and the new key and value if it holds slot p) go to LDS.
  __shared__ float qsum[(G + 2) * HD];
  const float* qv = row;   // the group's head vectors: q of head g*G + j at qv + j*HD ...
  const float* kn = row + (size_t)(a.Hq + g) * HD;
  const float* vn = row + (size_t)(a.Hq + a.Hkv + g) * HD;
  if (a.qkv_S > 0) {
    // every load first (one memory round trip), then the sums in split order
    const int nsum = (holds_p ? G + 2 : G) * HD;
    const size_t sstride = (size_t)a.B * a.Nqkv;
    const float* P = a.qkv_part + (size_t)b * a.Nqkv;
    constexpr int NT = 64 * MF_WAVES;
    constexpr int IT = ((G + 2) * HD + NT - 1) / NT;  // values per thread at most
    float pv[IT][GEMM_MAX_SPLIT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = min(tid + it * NT, nsum - 1);  // past nsum: a repeat, never stored
      const int hv = idx / HD, d = idx % HD;
      const int n = (hv < G ? (g * G + hv) : hv == G ? a.Hq + g : a.Hq + a.Hkv + g) * HD + d;
#pragma unroll
      for (int s2 = 0; s2 < GEMM_MAX_SPLIT; ++s2) pv[it][s2] = P[min(s2, a.qkv_S - 1) * sstride + n];
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = tid + it * NT;
      float v = pv[it][0];
#pragma unroll
      for (int s2 = 1; s2 < GEMM_MAX_SPLIT; ++s2)
        if (s2 < a.qkv_S) v = v + pv[it][s2];
      if (idx < nsum) qsum[idx] = v;
    }
    qv = qsum;
    kn = qsum + G * HD;
    vn = qsum + (G + 1) * HD;
  } else {
    qv = row + (size_t)g * G * HD;
  }
  if (tid < HD / 2) css[tid] = csv;
  __syncthreads();
  mf_prep_queries<HD, G>(qv, css, qs, tid, 64 * MF_WAVES);
  if (holds_p) {
    const int pc = p % ATTN_SPLIT;
    for (int d = tid; d < HD; d += 64 * MF_WAVES) {
      const bool fh = d < HD / 2;
      const uint16_t kw = f2bf_a(rope_pair(kn[d], kn[fh ? d + HD / 2 : d - HD / 2], css[fh ? d : d - HD / 2], fh));
      const uint16_t vw = f2bf_a(vn[d]);
      kvn[0][d] = kw;
      kvn[1][d] = vw;
      ((uint16_t*)a.kpool)[pbase + kfrag_off(pc, d, HD)] = kw;
      ((uint16_t*)a.vpool)[pbase + vfrag_off(pc, d, HD)] = vw;
    }
  }
  __syncthreads();

  if (active) {
    u32x4 bq[KK];
    mf_load_bq<HD, G>(qs, l16, g4, bq);
    const int kb = c * ATTN_SPLIT, ke = min(kb + ATTN_SPLIT, nk);
    const bool has_new = fused && p >= kb && p < kb + ATTN_SPLIT;
    // the new key replaces slot p's old contents
    if (has_new) {
      const int tp = (p - kb) >> 4, rp = (p - kb) & 15;
      const unsigned take = l16 == rp ? ~0u : 0u;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (t == tp) {
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            const u32x4 knr = *(const u32x4*)&kvn[0][kk * 32 + g4 * 8];
#pragma unroll
            for (int e = 0; e < 4; ++e) kr[t][kk][e] = (kr[t][kk][e] & ~take) | (knr[e] & take);
          }
        }
    }
    f32x4 sc[4];
    mf_scores<HD>(kr, bq, sc);

    // V is loaded once the scores are issued: the values are needed only
    // after the softmax, and the K fragments' registers are free by then
    u32x4 vf[2][DT];
    mf_load_v<HD>(vrs, foff, vf);
    // a chunk wholly below slot p needs no masking (a uniform branch)
    if (p < kb + ATTN_SPLIT) mf_mask_v<HD>(vf, kb, pk, has_new, p, g4, l16, kvn[1]);
    float o[4 / CPH][DT], m, l;
    mf_softmax_pv<HD, G>(sc, vf, kb, ke, g4, l16, o, m, l);
    mf_store_partial<HD, G>(o, m, l, g4, l16, os[w], ms[w], ls[w]);
  }
  __syncthreads();

  // The group's partial: every thread merges the chunks of its outputs in
  // chunk order.  A row with one partial is finished here.
  const bool direct = nk <= ATTN_SPLIT * ATTN_GROUP;
  const size_t pstride = (size_t)G * (HD + 2);
  float* dst = a.part + (((size_t)b * a.max_splits + c0 / ATTN_GROUP) * a.Hkv + g) * pstride;
  for (int idx = tid; idx < G * HD; idx += 64 * MF_WAVES) {
    const int j = idx / HD, d = idx % HD;
    const Merged r = merge_chunks(nc, &ms[0][j], &ls[0][j], G, &os[0][j][d], G * HD);
    if (direct) {
      put_out(a.out, (size_t)b * a.Hq * HD + (size_t)(g * G + j) * HD + d, r.o / r.l, WT_BF16);
    } else {
      dst[(size_t)j * (HD + 2) + d] = r.o;
      if (d == 0) {
        dst[(size_t)j * (HD + 2) + HD] = r.m;
        dst[(size_t)j * (HD + 2) + HD + 1] = r.l;
      }
    }
  }
}

// ---- batched prefill: many rows of one lane per work item ---------------------
//
// "parallel-slots.md" (section "Reuse: batched PREFILL already exists"): a
// prompt enters as many rows of one call.  Every row of a lane attends to
// the same cache, so one work item takes up to ATTN_ROWS_MAX consecutive rows of
// one lane (positions pa .. pa + nr - 1) and one aligned group of ATTN_GROUP
// chunks: each wave loads its chunk's K and V fragments once and keeps them
// in registers while it computes the chunk partial of every row that reaches
// it, with the same per-chunk code and merge as k_attn_mf (so a row's
// partial has the bits a decode step at that position gives).  Per row: the
// workgroup stores the next row's rotated, split queries into the other half
// of a double-buffered LDS area (their inputs loaded a row earlier), every
// wave writes its chunk partial, one barrier, and the row's group partial (or,
// for a row with one partial, its output) is merged and written.  Every row's key and value are in the cache
// already (k_kv_append runs first).
template <int HD, int G>
__global__ __launch_bounds__(64 * MF_WAVES) __attribute__((amdgpu_waves_per_eu(2))) void k_attn_rows(AttnArgs a) {
  constexpr int KK = HD / 32;
  constexpr int DT = HD / 16;
  constexpr int CPH = MfCols<G>::CPH;
  static_assert(ATTN_SPLIT == 64, "four 16-key tiles, two 32-key blocks");

  const int item = blockIdx.x / a.Hkv;  // item-major, as k_attn_mf
  if (item >= *a.n_items_dev) return;
  const int g = blockIdx.x % a.Hkv;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int4 it4 = *(const int4*)(a.items + ITEM_INTS * item);
  const int4 bl4 = *(const int4*)(a.items + ITEM_INTS * item + 4);
  const int first = it4.x & 0xffffff, nr = it4.x >> 24, c0 = it4.y, pa = it4.z, ncl = it4.w;
  const int* rows = a.rowmap + first;
  const int c = c0 + w;
  const bool loaded = w < ncl;  // some row of the item reaches this wave's chunk
  const long long hoff = a.layer_off + (long long)g * ATTN_SPLIT * HD;
  const int myblk = w == 0 ? bl4.x : w == 1 ? bl4.y : w == 2 ? bl4.z : bl4.w;
  const long long base = (long long)myblk * a.block_elems + hoff;
  const unsigned chunk_bytes = (unsigned)ATTN_SPLIT * HD * 2;
  const __amdgpu_buffer_rsrc_t krs = chunk_rsrc((const uint16_t*)a.kpool + base, chunk_bytes);
  const __amdgpu_buffer_rsrc_t vrs = chunk_rsrc((const uint16_t*)a.vpool + base, chunk_bytes);
  const unsigned foff = loaded ? (unsigned)lane * 16 : PAST_RANGE;
  u32x4 kr[4][KK], vf[2][DT];
  mf_load_k<HD>(krs, foff, kr);
  mf_load_v<HD>(vrs, foff, vf);

  __shared__ __attribute__((aligned(16))) uint16_t qs[2][16][HD];
  __shared__ float os[2][MF_WAVES][G][HD], ms[2][MF_WAVES][G], ls[2][MF_WAVES][G];
  __shared__ int rws[ATTN_ROWS_MAX];
  // The next row's query inputs are loaded one row ahead (registers) and
  // rotated, split and stored to the other LDS half one row ahead, so no row
  // waits on its own query loads.
  constexpr int NE = (G * HD + 64 * MF_WAVES - 1) / (64 * MF_WAVES);  // query elements per thread
  QIn qin[NE];
  auto qload = [&](int r) {
    const int b = rws[r];
    const float* qv = a.qkv + (size_t)b * a.Nqkv + (size_t)g * G * HD;
    const float2* cs = a.rope + (size_t)b * (HD / 2);
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const int idx = tid + e * 64 * MF_WAVES;
      if (idx < G * HD) qin[e] = mf_query_in<HD>(qv, cs, idx);
    }
  };
  auto qstore = [&](int buf) {
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const int idx = tid + e * 64 * MF_WAVES;
      if (idx < G * HD) mf_query_out<HD, G>(qin[e], idx, qs[buf]);
    }
  };
  if (tid < nr) rws[tid] = rows[tid];
  __syncthreads();
  qload(0);
  qstore(0);
  if (nr > 1) qload(1);
  __syncthreads();
  const size_t pstride = (size_t)G * (HD + 2);
  for (int r = 0; r < nr; ++r) {
    const int buf = r & 1;
    const int p = pa + r, nk = p + 1;
    const int ncr = min(ATTN_GROUP, p / ATTN_SPLIT + 1 - c0);  // the group's chunks this row reaches
    u32x4 bq[KK];
    mf_load_bq<HD, G>(qs[buf], l16, g4, bq);
    if (r + 1 < nr) qstore(buf ^ 1);
    if (r + 2 < nr) qload(r + 2);
    if (w < ncr) {
      const int kb = c * ATTN_SPLIT, ke = min(kb + ATTN_SPLIT, nk);
      f32x4 sc[4];
      mf_scores<HD>(kr, bq, sc);
      float o[4 / CPH][DT], m, l;
      if (p < kb + ATTN_SPLIT) {  // the row's last chunk: keys past p zeroed in a copy
        u32x4 vm[2][DT];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) vm[u][dt] = vf[u][dt];
        mf_mask_v<HD>(vm, kb, nk, false, p, g4, l16, nullptr);
        mf_softmax_pv<HD, G>(sc, vm, kb, ke, g4, l16, o, m, l);
      } else {
        mf_softmax_pv<HD, G>(sc, vf, kb, ke, g4, l16, o, m, l);
      }
      mf_store_partial<HD, G>(o, m, l, g4, l16, os[buf][w], ms[buf][w], ls[buf][w]);
    }
    __syncthreads();
    const int b = rws[r];
    const bool direct = nk <= ATTN_SPLIT * ATTN_GROUP;
    float* dst = a.part + (((size_t)b * a.max_splits + c0 / ATTN_GROUP) * a.Hkv + g) * pstride;
    for (int idx = tid; idx < G * HD; idx += 64 * MF_WAVES) {
      const int j = idx / HD, d = idx % HD;
      const Merged mr = merge_chunks(ncr, &ms[buf][0][j], &ls[buf][0][j], G, &os[buf][0][j][d], G * HD);
      if (direct) {
        put_out(a.out, (size_t)b * a.Hq * HD + (size_t)(g * G + j) * HD + d, mr.o / mr.l, WT_BF16);
      } else {
        dst[(size_t)j * (HD + 2) + d] = mr.o;
        if (d == 0) {
          dst[(size_t)j * (HD + 2) + HD] = mr.m;
          dst[(size_t)j * (HD + 2) + HD + 1] = mr.l;
        }
      }
    }
  }
}

// Every row's new key (rotated at the row's position) and value, rounded to
// the KV format, into slot pos[b] of its lane's block rowblk[b] (fragment
// order when a.frag is set); one workgroup per row, all KV heads.  The same
// rotation and rounding as the fused decode kernels.
template <bool BF>
__global__ __launch_bounds__(256) void k_kv_append(AttnArgs a, int hd) {
  const int b = blockIdx.x;
  const int p = a.pos[b];
  const int h = hd / 2, pc = p % ATTN_SPLIT;
  const long long base = (long long)a.rowblk[b] * a.block_elems + a.layer_off;
  const float* row = a.qkv + (size_t)b * a.Nqkv;
  const float2* cs = a.rope + (size_t)b * h;
  for (int e = threadIdx.x; e < a.Hkv * hd; e += blockDim.x) {
    const int g = e / hd, d = e % hd;
    const bool fh = d < h;
    const float* kn = row + (size_t)(a.Hq + g) * hd;
    const float k = rope_pair(kn[d], kn[fh ? d + h : d - h], cs[fh ? d : d - h], fh);
    const float v = row[(size_t)(a.Hq + a.Hkv + g) * hd + d];
    const long long cb = base + (long long)g * ATTN_SPLIT * hd;
    const long long ko = cb + (a.frag ? kfrag_off(pc, d, hd) : pc * hd + d);
    const long long vo = cb + (a.frag ? vfrag_off(pc, d, hd) : pc * hd + d);
    if constexpr (BF) {
      ((uint16_t*)a.kpool)[ko] = f2bf_a(k);
      ((uint16_t*)a.vpool)[vo] = f2bf_a(v);
    } else {
      ((float*)a.kpool)[ko] = k;
      ((float*)a.vpool)[vo] = v;
    }
  }
}

template <int ACT>
__device__ inline void put_act(void* base, size_t idx, float v) {
  if constexpr (ACT == WT_F32)
    ((float*)base)[idx] = v;
  else if constexpr (ACT == WT_BF16)
    ((uint16_t*)base)[idx] = f2bf_a(v);
  else
    ((_Float16*)base)[idx] = (_Float16)v;
}

// Combine a lane's partials (one per chunk, or per group of chunks):
// o = sum_s e^{m_s - M} o_s / sum_s e^{m_s - M} l_s, M = max_s m_s.  One
// thread per output (group head j, dim) of one (lane, KV head); it loads its
// partials in batches of COMB_BATCH (one memory round trip per batch) and adds
// them in partial order, so the result depends on the lane's position only.
constexpr int COMB_BATCH = 16;
constexpr int COMB_THREADS = 512;

template <int ACT>
__global__ __launch_bounds__(COMB_THREADS) void k_attn_combine(AttnArgs a, int hd) {
  const int b = blockIdx.x, g = blockIdx.y;
  const int e = blockIdx.z * blockDim.x + threadIdx.x;  // output j * hd + dim of the group
  if (b >= a.B || e >= a.G * hd) return;
  const int j = e / hd, dim = e % hd;
  const int nchunk = (a.pos[b] + 1 + ATTN_SPLIT - 1) / ATTN_SPLIT;
  const int ns = (nchunk + a.per - 1) / a.per;
  if (ns == 1) return;  // the attention kernel finished the row itself
  const size_t sstride = (size_t)a.Hkv * a.G * (hd + 2);
  const float* P = a.part + (((size_t)b * a.max_splits * a.Hkv + g) * a.G + j) * (hd + 2);
  float M = -INFINITY;
  if (ns > COMB_BATCH)  // more than one batch: the maximum over all partials first
    for (int s = 0; s < ns; ++s) M = fmaxf(M, P[(size_t)s * sstride + hd]);
  float O = 0.f, L = 0.f;
  for (int s0 = 0; s0 < ns; s0 += COMB_BATCH) {
    float mv[COMB_BATCH], ov[COMB_BATCH], lv[COMB_BATCH];
#pragma unroll
    for (int i = 0; i < COMB_BATCH; ++i) {
      const float* q = P + (size_t)min(s0 + i, ns - 1) * sstride;
      mv[i] = q[hd];
      lv[i] = q[hd + 1];
      ov[i] = q[dim];
    }
    if (ns <= COMB_BATCH) {
#pragma unroll
      for (int i = 0; i < COMB_BATCH; ++i)
        if (i < ns) M = fmaxf(M, mv[i]);
    }
#pragma unroll
    for (int i = 0; i < COMB_BATCH; ++i)
      if (s0 + i < ns) {
        const float w = expf(mv[i] - M);
        O += w * ov[i];
        L += w * lv[i];
      }
  }
  put_act<ACT>(a.out, (size_t)b * a.Hq * hd + (size_t)(g * a.G + j) * hd + dim, O / L);
}

// Waves of (item, KV head) below this count take one query head each: a
// wave's serial chain (scores, reduce-scatter, softmax, P.V of its heads)
// bounds a launch with few waves (SmolLM2-135M shape, 16-key contexts: 11.6
// -> 7.2 us at one lane, -6% per step at 64 lanes), while with more waves
// the repeated chunk loads cost more (+3% and +5% per step at 512 and 960
// lanes).  Splitting the group changes no result: each head is computed on
// its own.
constexpr long long ATTN_SPLIT_HEADS_BELOW = 512;

template <int HD, bool BF, int G>
static void launch_gk(const AttnArgs& a, dim3 grid, hipStream_t st) {
  const bool one = (long long)grid.x * grid.y < ATTN_SPLIT_HEADS_BELOW;
  const dim3 g2((unsigned)(((long long)grid.x + 7) / 8 * 8 * (one ? G : 1)), grid.y);
  if (one || G == 1)
    hipLaunchKernelGGL((k_attn<HD, BF, 1>), g2, dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL((k_attn<HD, BF, G>), g2, dim3(64), 0, st, a);
}

template <int HD, bool BF>
static hipError_t launch_g(int G, const AttnArgs& a, dim3 grid, hipStream_t st) {
  switch (G) {
    case 1: launch_gk<HD, BF, 1>(a, grid, st); break;
    case 2: launch_gk<HD, BF, 2>(a, grid, st); break;
    case 3: launch_gk<HD, BF, 3>(a, grid, st); break;
    case 4: launch_gk<HD, BF, 4>(a, grid, st); break;
    case 8: launch_gk<HD, BF, 8>(a, grid, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int HD>
static hipError_t launch_hd(int kv_bf16, int G, const AttnArgs& a, dim3 grid, hipStream_t st) {
  return kv_bf16 ? launch_g<HD, true>(G, a, grid, st) : launch_g<HD, false>(G, a, grid, st);
}

template <int HD>
static hipError_t launch_mf(int G, const AttnArgs& a, dim3 grid, hipStream_t st) {
  const dim3 blk(64 * MF_WAVES);
  switch (G) {
    case 1: hipLaunchKernelGGL((k_attn_mf<HD, 1>), grid, blk, 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_attn_mf<HD, 2>), grid, blk, 0, st, a); break;
    case 3: hipLaunchKernelGGL((k_attn_mf<HD, 3>), grid, blk, 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_attn_mf<HD, 4>), grid, blk, 0, st, a); break;
    case 5: case 6: case 7: case 8:
      if constexpr (HD == 64) {
        if (G == 5) hipLaunchKernelGGL((k_attn_mf<HD, 5>), grid, blk, 0, st, a);
        if (G == 6) hipLaunchKernelGGL((k_attn_mf<HD, 6>), grid, blk, 0, st, a);
        if (G == 7) hipLaunchKernelGGL((k_attn_mf<HD, 7>), grid, blk, 0, st, a);
        if (G == 8) hipLaunchKernelGGL((k_attn_mf<HD, 8>), grid, blk, 0, st, a);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn(int hd, int kv_bf16, const AttnArgs& a, hipStream_t st) {
  if (a.max_items <= 0) return hipSuccess;
  const dim3 grid(a.max_items, a.Hkv);
  if (attn_mfma_supported(hd, kv_bf16 != 0, a.G)) {
    const dim3 flat((unsigned)a.max_items * a.Hkv);
    return hd == 128 ? launch_mf<128>(a.G, a, flat, st) : launch_mf<64>(a.G, a, flat, st);
  }
  switch (hd) {
    case 16: return launch_hd<16>(kv_bf16, a.G, a, grid, st);
    case 32: return launch_hd<32>(kv_bf16, a.G, a, grid, st);
    case 64: return launch_hd<64>(kv_bf16, a.G, a, grid, st);
    case 128: return launch_hd<128>(kv_bf16, a.G, a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

template <int HD>
static hipError_t launch_rows_hd(int G, const AttnArgs& a, dim3 grid, hipStream_t st) {
  const dim3 blk(64 * MF_WAVES);
  switch (G) {
    case 1: hipLaunchKernelGGL((k_attn_rows<HD, 1>), grid, blk, 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_attn_rows<HD, 2>), grid, blk, 0, st, a); break;
    case 3: hipLaunchKernelGGL((k_attn_rows<HD, 3>), grid, blk, 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_attn_rows<HD, 4>), grid, blk, 0, st, a); break;
    case 5: case 6: case 7: case 8:
      if constexpr (HD == 64) {
        if (G == 5) hipLaunchKernelGGL((k_attn_rows<HD, 5>), grid, blk, 0, st, a);
        if (G == 6) hipLaunchKernelGGL((k_attn_rows<HD, 6>), grid, blk, 0, st, a);
        if (G == 7) hipLaunchKernelGGL((k_attn_rows<HD, 7>), grid, blk, 0, st, a);
        if (G == 8) hipLaunchKernelGGL((k_attn_rows<HD, 8>), grid, blk, 0, st, a);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_rows(int hd, const AttnArgs& a, hipStream_t st) {
  if (a.max_items <= 0) return hipSuccess;
  if (!attn_mfma_supported(hd, true, a.G)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)a.max_items * a.Hkv);
  return hd == 128 ? launch_rows_hd<128>(a.G, a, grid, st) : launch_rows_hd<64>(a.G, a, grid, st);
}

hipError_t launch_kv_append(int hd, int kv_bf16, const AttnArgs& a, hipStream_t st) {
  if (a.B <= 0) return hipSuccess;
  if (kv_bf16)
    hipLaunchKernelGGL(k_kv_append<true>, dim3(a.B), dim3(256), 0, st, a, hd);
  else
    hipLaunchKernelGGL(k_kv_append<false>, dim3(a.B), dim3(256), 0, st, a, hd);
  return hipGetLastError();
}

hipError_t launch_attn_combine(int hd, int act, const AttnArgs& a, hipStream_t st) {
  if (a.max_items <= 0) return hipSuccess;
  if (a.G > 8) return hipErrorInvalidValue;
  const int nthr = std::min(COMB_THREADS, (a.G * hd + 63) / 64 * 64);
  const dim3 cgrid(a.B, a.Hkv, (a.G * hd + nthr - 1) / nthr);
  const dim3 blk(nthr);
  switch (act) {
    case WT_F32: hipLaunchKernelGGL(k_attn_combine<WT_F32>, cgrid, blk, 0, st, a, hd); break;
    case WT_BF16: hipLaunchKernelGGL(k_attn_combine<WT_BF16>, cgrid, blk, 0, st, a, hd); break;
    default: hipLaunchKernelGGL(k_attn_combine<WT_Q8>, cgrid, blk, 0, st, a, hd); break;
  }
  return hipGetLastError();
}

}  // namespace cbd
