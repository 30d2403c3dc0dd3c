// mk_device.hip - the persistent decode interpreter and its op bodies (gfx950).
//
// One workgroup of 512 threads (8 wave64s) stays resident per compute unit
// and walks its host-built task list (Cohere North Mini Code megakernel post,
// section "What is a Megakernel?"). Each task:
//   1. issues the loads of its weight tiles (weights do not depend on this
//      step's activations, so they stream before the dependency clears:
//      section "Weight prefetch");
//   2. spins until its input counters reach their targets (the barrier
//      listing of the Chinese version: spin on a global counter, then fence);
//   3. computes and stores its output tile;
//   4. makes its stores visible at device scope and increments its output
//      counter (release, then atomic add).
// The same kernel, launched once per wave of same-type tasks with waits
// switched off, is the kernel-per-op variant.
//
// Memory ordering on CDNA4. Each XCD has its own L2, which is not coherent with
// the other XCDs' L2s. A C++ release/acquire at agent scope is implemented by
// writing back / invalidating the whole L2 (buffer_wbl2 / buffer_inv), which
// costs microseconds per task, so the interpreter does not use them. Instead
// every activation that crosses compute units within a step is stored and
// loaded with device-scope (sc1) buffer instructions, which bypass the
// non-coherent cache levels; a producer waits for its own stores to complete
// (s_waitcnt) before its counter increment, and a consumer issues its loads
// only after it has observed the counter. Weights and the KV cache written in
// earlier steps are read with ordinary (non-temporal) loads: nothing writes
// them during a step, and kernel boundaries make earlier steps' writes visible.
#include <hip/hip_runtime.h>

#include "mk_internal.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

namespace {

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// Wave index as a scalar (wave-uniform) value, so per-wave chunk choices
// compile to scalar branches instead of exec-mask juggling.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
// float -> bf16 bits, round to nearest even
__device__ __forceinline__ uint32_t f2bf(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Raw buffer resource over a uniform base address (4 GB range). Loads past
// the range return 0 instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, -1, 0x00020000);
}
constexpr int kSC1 = 16;  // cache-policy bit: device (agent) scope coherence

// Device-coherent access to a buffer of 32-bit words shared across compute units.
struct Pub {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ explicit Pub(const void* base) : r(rsrc_of(base)) {}
  __device__ __forceinline__ float ldf(int i) const {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, i * 4, 0, kSC1));
  }
  __device__ __forceinline__ int ldi(int i) const {
    return (int)__builtin_amdgcn_raw_buffer_load_b32(r, i * 4, 0, kSC1);
  }
  __device__ __forceinline__ float4 ldf4(int i) const {  // 16-byte aligned element index
    // (element values through __uint_as_float: a bit-cast of an ext-vector
    // element would read the vector's first element)
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, i * 4, 0, kSC1);
    return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
  }
  __device__ __forceinline__ void stf(int i, float v) const {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, i * 4, 0, kSC1);
  }
  __device__ __forceinline__ void sti(int i, int v) const {
    __builtin_amdgcn_raw_buffer_store_b32((uint32_t)v, r, i * 4, 0, kSC1);
  }
  __device__ __forceinline__ void st16(int i, uint16_t v) const {  // i: 16-bit element index
    __builtin_amdgcn_raw_buffer_store_b16(v, r, i * 2, 0, kSC1);
  }
  __device__ __forceinline__ u32x4_t ld16x8(int i) const {  // 8 bf16 at 16-bit index i
    return __builtin_amdgcn_raw_buffer_load_b128(r, i * 2, 0, kSC1);
  }
  __device__ __forceinline__ u32x2_t ld16x4(int i) const {  // 4 bf16 at 16-bit index i
    return __builtin_amdgcn_raw_buffer_load_b64(r, i * 2, 0, kSC1);
  }
};

// Wait until this wave's memory operations have completed.
__device__ __forceinline__ void drain_memory() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("" ::: "memory");
}

// Workgroup barrier after which device-coherent stores of every wave are complete.
__device__ __forceinline__ void sync_published() {
  drain_memory();
  __syncthreads();
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

constexpr float kNegInf = -__builtin_inff();

struct SmemAttn {
  float m[MK_WAVES][16];
  float l[MK_WAVES][16];
  float o[MK_WAVES][128][17];
};

// Attention combine scratch: per split and head, the rescale factor.
#define MK_MAX_SPLITS 256
struct SmemComb {
  float f[MK_MAX_SPLITS][16];
  float l[MK_MAX_SPLITS][16];
  float M[16];
  float L[16];
};

// LDS per workgroup: with one workgroup per compute unit, more than half of
// gfx950's 160 KB (so exactly one fits); with two, more than a third.
struct SmemTopk {
  alignas(16) float logit[128];
  float sel_val[MK_MAX_TOPK];
  int sel_idx[MK_MAX_TOPK];
};

union SmemU {
  float red[MK_WAVES][64];
  SmemTopk tk;
  SmemAttn at;
  SmemComb cb;
  float pad[MK_WGS_PER_CU == 1 ? 20480 : 11264];
};

// Arrays read as float4 must be 16-byte aligned: a 16-byte LDS read from a
// 4-byte aligned address runs about five times slower on gfx950 (a 64-chunk
// GEMV over an LDS vector measured 3.7 us unaligned against 0.7 us aligned).
struct Smem {
  SmemU u;
  alignas(16) float out[64];
  alignas(16) float ssq[128];
  alignas(16) float xc[2048];  // normalised input of one layer for batch 1 (per compute unit)
  alignas(16) float us[768];   // expert hidden of one routed slot (down projection input)
  alignas(16) float vred[MK_WAVES];
  int ired[MK_WAVES];
  int flag;
  int claim;
  int old;                // value an arrival counter held before this workgroup's increment
  uint32_t t_waited;
  uint32_t t_mark[4];     // op-defined intermediate timestamps (e.g. inputs ready, computed)
  int xc_layer;           // layer whose normalised input xc holds (-1: none)
  int rt_hdr[4];          // route header: n_active, up items, down items
  int rt_e[128];          // active experts, ascending
  int rt_slot[128];       // batch 1: the routed slot of each active expert
};
static_assert(offsetof(Smem, xc) % 16 == 0 && offsetof(Smem, us) % 16 == 0 &&
              offsetof(Smem, out) % 16 == 0 && offsetof(Smem, ssq) % 16 == 0, "LDS vectors 16-byte aligned");

__device__ void raise_error(const mk_params& P, uint32_t code, uint32_t detail, uint32_t value) {
  uint32_t expected = 0;
  if (__hip_atomic_compare_exchange_strong(&P.err[0], &expected, code, __ATOMIC_RELAXED,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
    __hip_atomic_store(&P.err[1], detail, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&P.err[2], value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&P.err[3], (uint32_t)blockIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Spin (thread 0) until ctr[c] >= tgt for each wait, or until another
// workgroup raised an error, or until the time limit. Block-uniform result.
__device__ bool wait_counters(const mk_params& P, const int32_t* cs, const int32_t* ts, int n, Smem& sm) {
  if (threadIdx.x == 0) {
    int ok = ld_relaxed(&P.err[0]) == 0;
    if (ok && P.waits_enabled) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      for (int i = 0; i < n && ok; ++i) {
        if (cs[i] < 0) continue;
        const uint32_t* c = P.ctr + cs[i];
        const uint32_t tgt = (uint32_t)ts[i];
        uint32_t spins = 0;
        while (ld_relaxed(c) < tgt) {
          __builtin_amdgcn_s_sleep(2);
          if ((++spins & 63u) == 0) {
            if (ld_relaxed(&P.err[0]) != 0) { ok = 0; break; }
            if ((int64_t)(__builtin_amdgcn_s_memrealtime() - t0) > P.timeout_ticks) {
              raise_error(P, MK_DEVERR_TIMEOUT, (uint32_t)cs[i], ld_relaxed(c));
              ok = 0;
              break;
            }
          }
        }
      }
    }
    sm.flag = ok;
    sm.t_waited = (uint32_t)__builtin_amdgcn_s_memrealtime();
  }
  __syncthreads();
  const bool ok = sm.flag != 0;
  __syncthreads();
  return ok;
}

__device__ __forceinline__ bool wait_task(const mk_params& P, const mk_task& t, Smem& sm) {
  return wait_counters(P, t.wait_ctr, t.wait_tgt, 3, sm);
}

__device__ __forceinline__ bool wait_one(const mk_params& P, int32_t c, int32_t tgt, Smem& sm) {
  return wait_counters(P, &c, &tgt, 1, sm);
}

__device__ __forceinline__ int layer_window(const mk_params& P, int l) {
  if (P.window == 0) return 0;
  return (l % P.full_every) == P.full_every - 1 ? 0 : P.window;
}

// ----------------------------------------------------- batch-1 GEMV panels
//
// Weight matrices [K x N] are stored panel-tiled: 16-column panels, each a run
// of K/32 chunks of 1 KB; in a chunk, lane l holds the 8 bf16 of rows
// 32c + 8(l/16) + i (i = 0..7) of column 16j + l%16. Chunk c of a panel goes
// to wave c % 8, so each wave keeps its slice of the activation vector in
// registers and every load is one contiguous 1 KB line per wave.

template <int NP, int NCH>
struct WTile {
  u32x4_t v[NP][NCH];
};

// Chunks outside [c0, c1) and panels at or beyond np are zero, so the GEMVs
// below run without per-chunk branches.
template <int NP, int NCH>
__device__ __forceinline__ void wtile_load(WTile<NP, NCH>& w, const uint16_t* base, size_t pstride,
                                           int np, int c0, int c1) {
  const int wv = wave_id(), ln = lane_id();
#pragma unroll
  for (int pp = 0; pp < NP; ++pp)
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = c0 + wv + MK_WAVES * i;
      if (pp < np && c < c1)
        w.v[pp][i] = __builtin_nontemporal_load((const u32x4_t*)(base + pp * pstride + (size_t)c * 512) + ln);
      else
        w.v[pp][i] = u32x4_t{0u, 0u, 0u, 0u};
    }
}

__device__ __forceinline__ float dot8(float4 x0, float4 x1, u32x4_t q, float s) {
  s = fmaf(x0.x, bf_lo(q.x), s);
  s = fmaf(x0.y, bf_hi(q.x), s);
  s = fmaf(x0.z, bf_lo(q.y), s);
  s = fmaf(x0.w, bf_hi(q.y), s);
  s = fmaf(x1.x, bf_lo(q.z), s);
  s = fmaf(x1.y, bf_hi(q.z), s);
  s = fmaf(x1.z, bf_lo(q.w), s);
  s = fmaf(x1.w, bf_hi(q.w), s);
  return s;
}

// y[16*pp + col] = sum_k x[k - 32*c0] * W[k][col] over chunks [c0, c1), into sm.out.
// x: float32 activations (another compute unit's output) starting at row 32*c0.
template <int NP, int NCH>
__device__ void gemv_b1(const WTile<NP, NCH>& w, const float* x, int np, int c0, int c1, Smem& sm) {
  const Pub X(x);
  const int wv = wave_id(), ln = lane_id();
  float acc[NP];
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) acc[pp] = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    // out-of-range chunks read a valid row and multiply zero weights
    const int c = max(min(c0 + wv + MK_WAVES * i, c1 - 1), c0);
    const int xi = (c - c0) * 32 + 8 * (ln >> 4);
    const float4 x0 = X.ldf4(xi), x1 = X.ldf4(xi + 4);
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) acc[pp] = dot8(x0, x1, w.v[pp][i], acc[pp]);
  }
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) {
    acc[pp] += __shfl_xor(acc[pp], 16);
    acc[pp] += __shfl_xor(acc[pp], 32);
  }
  if (ln < 16) {
#pragma unroll
    for (int pp = 0; pp < NP; ++pp)
      if (pp < np) sm.u.red[wv][pp * 16 + ln] = acc[pp];
  }
  __syncthreads();
  if (threadIdx.x < np * 16) {
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < MK_WAVES; ++k) s += sm.u.red[k][threadIdx.x];
    sm.out[threadIdx.x] = s;
  }
  __syncthreads();
}

__device__ __forceinline__ void mark(Smem& sm, int k) {
  if (threadIdx.x == 0) sm.t_mark[k] = (uint32_t)__builtin_amdgcn_s_memrealtime();
}

// ---------------------------------------------------------- arrivals
// Count one arrival on counter c once every wave's device-coherent stores
// have completed.
__device__ void arrive_nr(const mk_params& P, int32_t c) {
  sync_published();
  if (threadIdx.x == 0 && c >= 0)
    __hip_atomic_fetch_add(&P.ctr[c], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The same, returning (block-uniform) the value the counter held before this
// arrival, so the last of a known number of arrivals can act on the result.
__device__ int arrive(const mk_params& P, int32_t c, Smem& sm) {
  sync_published();
  if (threadIdx.x == 0)
    sm.old = (int)__hip_atomic_fetch_add(&P.ctr[c], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int old = sm.old;
  __syncthreads();
  return old;
}

// ----------------------------------------------------- layer input x-hat
// The normalised input of layer l (megakernel post, section "Reduce wave
// quantization": attention and the MoE both read the same RMS-normalised
// input). Layer 0's residual is the token's embedding row; later layers'
// residual stream h is complete once every column block's residual add has
// arrived, each block leaving its sum of squares in ssq. Every compute unit
// forms x = h / sqrt(mean(h^2) + eps) * gamma_l once per layer into LDS
// (batch 1), so the fused residual + RMSNorm needs no task of its own.
__device__ bool load_xhat(const mk_params& P, int l, Smem& sm) {
  if (sm.xc_layer == l) return true;
  const int H = P.H;
  const uint16_t* gam = P.gamma + (size_t)l * H;
  constexpr int NV = 2048 / MK_WG_THREADS;  // H <= 2048
  float v[NV];
  float ss = 0.f;
  if (l == 0) {
    int tok = P.tokens[0];
    if (tok < 0 || tok >= P.V) {
      if (threadIdx.x == 0) raise_error(P, MK_DEVERR_FAULT, 1000, (uint32_t)tok);
      tok = 0;
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int i = threadIdx.x + k * MK_WG_THREADS;
      v[k] = i < H ? bf2f(P.emb[(size_t)tok * H + i]) : 0.f;
      ss = fmaf(v[k], v[k], ss);
    }
    ss = wave_sum(ss);
    if (lane_id() == 0) sm.vred[wave_id()] = ss;
  } else {
    const Pub h(P.h), q(P.ssq);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int i = threadIdx.x + k * MK_WG_THREADS;
      v[k] = i < H ? h.ldf(i) : 0.f;
    }
    if (threadIdx.x < P.NB) sm.ssq[threadIdx.x] = q.ldf(threadIdx.x);
  }
  __syncthreads();
  float tot = 0.f;
  if (l == 0) {
#pragma unroll
    for (int k = 0; k < MK_WAVES; ++k) tot += sm.vred[k];
  } else {
    for (int k = 0; k < P.NB; ++k) tot += sm.ssq[k];
  }
  const float inv = 1.0f / sqrtf(tot / (float)H + P.eps);
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int i = threadIdx.x + k * MK_WG_THREADS;
    if (i < H) sm.xc[i] = v[k] * inv * bf2f(gam[i]);
  }
  __syncthreads();
  if (threadIdx.x == 0) sm.xc_layer = l;
  __syncthreads();
  return true;
}

// gemv with x from the LDS copy of x-hat (rows 32*c0 .. of the layer input)
template <int NP, int NCH>
__device__ void gemv_lds(const WTile<NP, NCH>& w, const float* xl, int np, int c0, int c1, Smem& sm) {
  const int wv = wave_id(), ln = lane_id();
  float acc[NP];
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) acc[pp] = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    // out-of-range chunks read a valid row and multiply zero weights
    const int c = max(min(c0 + wv + MK_WAVES * i, c1 - 1), c0);
    const float4* xp = (const float4*)(xl + c * 32 + 8 * (ln >> 4));
    const float4 x0 = xp[0], x1 = xp[1];
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) acc[pp] = dot8(x0, x1, w.v[pp][i], acc[pp]);
  }
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) {
    acc[pp] += __shfl_xor(acc[pp], 16);
    acc[pp] += __shfl_xor(acc[pp], 32);
  }
  if (ln < 16) {
#pragma unroll
    for (int pp = 0; pp < NP; ++pp)
      if (pp < np) sm.u.red[wv][pp * 16 + ln] = acc[pp];
  }
  __syncthreads();
  if (threadIdx.x < np * 16) {
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < MK_WAVES; ++k) s += sm.u.red[k][threadIdx.x];
    sm.out[threadIdx.x] = s;
  }
  __syncthreads();
}

// -------------------------------------------------------------------- QKV
// QKV panels with RoPE in the epilogue and the K/V append into the paged
// cache (megakernel post, section "Tasks": QKV_PROJ applies RoPE in-register
// in its epilogue; tiny-vllm walkthrough: the new token's K/V are written to
// page block_table[pos / 16], slot pos % 16, before attention reads them).
template <int NCH>
__device__ __forceinline__ void op_qkv(const mk_params& P, const mk_task& t, Smem& sm) {
  const int l = t.layer, p0 = t.a[0], np = t.a[1];
  const int kc = P.H / 32;
  const size_t pstride = (size_t)kc * 512;
  WTile<2, NCH> w;  // up to two panels per task
  wtile_load(w, P.wqkv + l * P.s_wqkv + (size_t)p0 * pstride, pstride, np, 0, kc);
  if (!wait_task(P, t, sm)) return;
  load_xhat(P, l, sm);
  mark(sm, 0);
  const int qd = P.QH * P.D, kvd = P.KVH * P.D, D = P.D, PS = P.PS;
  gemv_lds(w, sm.xc, np, 0, kc, sm);
  mark(sm, 1);
  if (wave_id() == 0) {
    const int tid = threadIdx.x;
    const float y = tid < np * 16 ? sm.out[tid] : 0.f;
    const float yp = __shfl_xor(y, 1);
    const int seq = P.seq_lens[0];
    if (tid < np * 16) {
      if (seq < 1 || seq > P.max_seq) {
        if (tid == 0) raise_error(P, MK_DEVERR_FAULT, 2000, (uint32_t)seq);
      } else {
        const int pos = seq - 1;
        const int n = p0 * 16 + tid;
        const bool odd = n & 1;
        const int page = P.bt[pos / PS];
        const bool page_ok = page >= 0 && page < P.n_pages;
        if (n < qd + kvd) {
          const int d = (n < qd ? n : n - qd) % D;
          const float c = P.rope[((size_t)pos * (D / 2) + d / 2) * 2 + 0];
          const float s = P.rope[((size_t)pos * (D / 2) + d / 2) * 2 + 1];
          // pair (x0, x1) -> (x0 c - x1 s, x0 s + x1 c)
          const float x0 = odd ? yp : y, x1 = odd ? y : yp;
          const float r = odd ? (x0 * s + x1 * c) : (x0 * c - x1 * s);
          if (n < qd) {
            Pub(P.q).stf(n, r);
          } else if (page_ok) {
            const int g = (n - qd) / D;
            const int off = ((page * 2 + 0) * P.KVH + g) * PS * D + (pos % PS) * D + d;
            Pub(P.kv + l * P.s_kv_l).st16(off, (uint16_t)f2bf(r));
          }
        } else if (page_ok) {
          const int nn = n - qd - kvd;
          const int g = nn / D, d = nn % D;
          const int off = ((page * 2 + 1) * P.KVH + g) * PS * D + d * PS + (pos % PS);
          Pub(P.kv + l * P.s_kv_l).st16(off, (uint16_t)f2bf(y));
        }
        if (!page_ok && tid == 0) raise_error(P, MK_DEVERR_FAULT, 3000, (uint32_t)page);
      }
    }
  }
  arrive_nr(P, t.sig_ctr[0]);
}

// -------------------------------------------------------------- attention
// Split-KV partial attention of the G query heads of one kv group over a
// range of pages (megakernel post, section "Tasks": ATTN_DECODE over partial
// KV slices). MFMA with the keys as rows: S^T = K Q^T (16 keys x 16 heads per
// page, heads >= G padded), online softmax per head, O^T += V^T P^T (V is
// stored transposed within a page so each lane's operand is 8 contiguous
// bytes). The 8 waves take alternate pages and merge at the end; each wave's
// first page streams before the dependency wait (the older KV is immutable
// this step). The split that completes a (sequence, group) merges all splits
// (ATTN_COMBINE) without a task of its own.
template <int D>
__device__ void attn_combine(const mk_params& P, int b, int g, int ns, Smem& sm);

// One wave's operands of one KV page of one kv group: K rows (keys) for the
// score MFMA, V^T tiles for the output MFMA.
template <int D>
struct KVPage {
  u32x4_t k[D / 32];
  u32x2_t v[D / 16];
};

template <int D>
__device__ __forceinline__ void op_attn(const mk_params& P, const mk_task& t, Smem& sm) {
  constexpr int NC = D / 32;
  constexpr int NT = D / 16;
  const int l = t.layer, b = t.a[0], g = t.a[1], s = t.a[2], ns = t.a[3], pps = t.a[4];
  const int wv = wave_id(), ln = lane_id();
  const int PS = P.PS, G = P.G;
  const int seq = P.seq_lens[b];
  const bool seq_ok = seq >= 1 && seq <= P.max_seq;
  const int p = seq_ok ? seq - 1 : 0;
  const int win = layer_window(P, l);
  const int lo = win ? max(0, p - win + 1) : 0;
  const int lp_first = lo / PS, lp_last = p / PS;
  const int my0 = lp_first + s * pps;
  const int my1 = seq_ok ? min(my0 + pps, lp_last + 1) : my0;
  const uint16_t* kvl = P.kv + l * P.s_kv_l;
  const size_t plane = (size_t)PS * D;
  const float scale = P.attn_scale;

  bool bad = false;
  // The page holding the current position gets this step's K/V from the QKV
  // tasks of other compute units: read it device-coherently, after the wait.
  const Pub KV(kvl);
  auto load_page = [&](int lp) {
    KVPage<D> pg;
    const int phys = P.bt[b * P.mpps + lp];
    if (phys < 0 || phys >= P.n_pages) {
      bad = true;
      return pg;
    }
    const int ko = ((phys * 2 + 0) * P.KVH + g) * (int)plane, vo = ((phys * 2 + 1) * P.KVH + g) * (int)plane;
    if (lp == lp_last) {
#pragma unroll
      for (int c = 0; c < NC; ++c) pg.k[c] = KV.ld16x8(ko + (ln & 15) * D + 32 * c + 8 * (ln >> 4));
#pragma unroll
      for (int d = 0; d < NT; ++d) pg.v[d] = KV.ld16x4(vo + (16 * d + (ln & 15)) * PS + 4 * (ln >> 4));
    } else {
      const uint16_t* kp = kvl + ko;
      const uint16_t* vp = kvl + vo;
#pragma unroll
      for (int c = 0; c < NC; ++c)
        pg.k[c] = __builtin_nontemporal_load((const u32x4_t*)(kp + (ln & 15) * D + 32 * c + 8 * (ln >> 4)));
#pragma unroll
      for (int d = 0; d < NT; ++d)
        pg.v[d] = __builtin_nontemporal_load((const u32x2_t*)(vp + (16 * d + (ln & 15)) * PS + 4 * (ln >> 4)));
    }
    return pg;
  };

  // each wave's first two pages stream before the wait (two-deep pipeline)
  int lp = my0 + wv;
  const int lpn = lp + MK_WAVES;
  const bool early0 = lp < my1 && lp != lp_last, early1 = lpn < my1 && lpn != lp_last;
  KVPage<D> cur, nxt;
  if (early0) cur = load_page(lp);
  if (early1) nxt = load_page(lpn);
  if (!wait_task(P, t, sm)) return;
  if (!seq_ok) {
    if (threadIdx.x == 0) raise_error(P, MK_DEVERR_FAULT, 4000 + b, (uint32_t)seq);
    return;
  }
  if (lp < my1 && !early0) cur = load_page(lp);
  if (lpn < my1 && !early1) nxt = load_page(lpn);

  // Q^T operand: lane holds q[head ln%16][dims 32c + 8(ln/16) + i]
  bf16x8_t qb[NC];
  {
    const int hh = ln & 15;
    const Pub Q(P.q + (size_t)b * P.QH * D + (size_t)g * G * D);
    const int qo = min(hh, G - 1) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float4 a0 = Q.ldf4(qo + 32 * c + 8 * (ln >> 4)), a1 = Q.ldf4(qo + 32 * c + 8 * (ln >> 4) + 4);
      const float qv[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      u32x4_t pk;
#pragma unroll
      for (int i = 0; i < 4; ++i) pk[i] = hh < G ? (f2bf(qv[2 * i]) | (f2bf(qv[2 * i + 1]) << 16)) : 0u;
      qb[c] = __builtin_bit_cast(bf16x8_t, pk);
    }
  }

  f32x4_t oacc[NT];
#pragma unroll
  for (int d = 0; d < NT; ++d) oacc[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, lsum = 0.f;

  while (lp < my1 && !bad) {
    KVPage<D> nxt2;
    const int nlp2 = lp + 2 * MK_WAVES;
    if (nlp2 < my1) nxt2 = load_page(nlp2);
    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, cur.k[c]), qb[c], sacc, 0, 0, 0);
    float sv[4];
    float mloc = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pos = lp * PS + 4 * (ln >> 4) + i;
      sv[i] = (pos >= lo && pos <= p) ? sacc[i] * scale : kNegInf;
      mloc = fmaxf(mloc, sv[i]);
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float mnew = fmaxf(m, mloc);
    if (mnew != kNegInf) {
      const float alpha = (m == kNegInf) ? 0.f : __expf(m - mnew);
      uint32_t pb[4];
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = sv[i] == kNegInf ? 0.f : __expf(sv[i] - mnew);
        pb[i] = f2bf(pv);
        ps += bf2f((uint16_t)pb[i]);
      }
      ps += __shfl_xor(ps, 16);
      ps += __shfl_xor(ps, 32);
      lsum = lsum * alpha + ps;
      m = mnew;
      const s16x4_t pB = {(short)pb[0], (short)pb[1], (short)pb[2], (short)pb[3]};
#pragma unroll
      for (int d = 0; d < NT; ++d) {
        oacc[d] *= alpha;
        oacc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, cur.v[d]), pB, oacc[d], 0, 0, 0);
      }
    }
    cur = nxt;
    nxt = nxt2;
    lp += MK_WAVES;
  }
  if (bad) raise_error(P, MK_DEVERR_FAULT, 5000 + b, (uint32_t)lp);

  // merge the 8 waves' (m, l, O) per head into this split's partial
  SmemAttn& A = sm.u.at;
  if (ln < 16) {
    A.m[wv][ln] = m;
    A.l[wv][ln] = lsum;
  }
#pragma unroll
  for (int d = 0; d < NT; ++d)
#pragma unroll
    for (int i = 0; i < 4; ++i) A.o[wv][16 * d + 4 * (ln >> 4) + i][ln & 15] = oacc[d][i];
  __syncthreads();
  const int stride = G * D + 2 * G;
  const Pub dst(P.part + ((size_t)(b * P.KVH + g) * P.max_splits + s) * stride);
  for (int idx = threadIdx.x; idx < G * D; idx += MK_WG_THREADS) {
    const int hh = idx / D, dd = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int k = 0; k < MK_WAVES; ++k) M = fmaxf(M, A.m[k][hh]);
    float O = 0.f, L = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int k = 0; k < MK_WAVES; ++k) {
        const float f = A.m[k][hh] == kNegInf ? 0.f : __expf(A.m[k][hh] - M);
        O = fmaf(f, A.o[k][dd][hh], O);
        L = fmaf(f, A.l[k][hh], L);
      }
    }
    dst.stf(hh * D + dd, O);
    if (dd == 0) {
      dst.stf(G * D + hh, M);
      dst.stf(G * D + G + hh, L);
    }
  }
  mark(sm, 0);
  const int old = arrive(P, t.a[5], sm);
  mark(sm, 1);
  if (old == ns - 1) {
    attn_combine<D>(P, b, g, ns, sm);
    mark(sm, 3);
    arrive_nr(P, t.sig_ctr[0]);
  }
}

// Log-sum-exp merge of one (sequence, kv group)'s split partials into the
// attention output (megakernel post, section "Tasks": ATTN_COMBINE):
// o = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s, splits in fixed order.
template <int D>
__device__ void attn_combine(const mk_params& P, int b, int g, int ns, Smem& sm) {
  const int G = P.G;
  const int stride = G * D + 2 * G;
  const Pub src(P.part + (size_t)(b * P.KVH + g) * P.max_splits * stride);
  SmemComb& C = sm.u.cb;
  // split maxima and sums, all loads in flight together
  for (int i = threadIdx.x; i < ns * G; i += MK_WG_THREADS) {
    const int s = i / G, hh = i % G;
    C.f[s][hh] = src.ldf(s * stride + G * D + hh);
    C.l[s][hh] = src.ldf(s * stride + G * D + G + hh);
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int hh = threadIdx.x;
    float M = kNegInf;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, C.f[s][hh]);
    C.M[hh] = M;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < ns * G; i += MK_WG_THREADS) {
    const int s = i / G, hh = i % G;
    const float ms = C.f[s][hh];
    C.f[s][hh] = ms == kNegInf ? 0.f : __expf(ms - C.M[hh]);
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int hh = threadIdx.x;
    float L = 0.f;
    for (int s = 0; s < ns; ++s) L = fmaf(C.f[s][hh], C.l[s][hh], L);
    C.L[hh] = L;
  }
  __syncthreads();
  mark(sm, 2);
  const Pub dst(P.o + (size_t)b * P.QH * D + (size_t)g * G * D);
  // each thread's outputs (G * D <= 1024: at most two) over up to 32 splits
  // at a time, every load in flight together
  constexpr int NO = 1024 / MK_WG_THREADS, SB = 32;
  float O[NO];
#pragma unroll
  for (int u = 0; u < NO; ++u) O[u] = 0.f;
  for (int s0 = 0; s0 < ns; s0 += SB) {
    float v[NO][SB];
#pragma unroll
    for (int u = 0; u < NO; ++u) {
      const int idx = threadIdx.x + u * MK_WG_THREADS;
      const int hh = idx / D, dd = idx % D;
#pragma unroll
      for (int k = 0; k < SB; ++k)
        v[u][k] = (idx < G * D && s0 + k < ns) ? src.ldf((s0 + k) * stride + hh * D + dd) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < NO; ++u) {
      const int idx = threadIdx.x + u * MK_WG_THREADS;
      const int hh = min(idx / D, G - 1);
#pragma unroll
      for (int k = 0; k < SB; ++k)
        if (s0 + k < ns) O[u] = fmaf(C.f[s0 + k][hh], v[u][k], O[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < NO; ++u) {
    const int idx = threadIdx.x + u * MK_WG_THREADS;
    if (idx < G * D) dst.stf(idx, O[u] / C.L[idx / D]);
  }
}

// ------------------------------------------------------------- residual
// Residual add of one column block, done by whichever contribution to the
// block arrives last (the KVH O-projection partials and the block's tile of
// every routed expert's down projection): h += sum_g a_g + sum_j w_j y_j,
// the experts summed in rank order (MOE_COMBINE), then the block's sum of
// squares for the next layer's RMSNorm. Layer 0 adds to the embedding row.
__device__ void residual_block(const mk_params& P, int l, int cb, Smem& sm) {
  const int H = P.H, K = P.K, CB = P.CB;
  const Pub h(P.h), ao(P.ao), dn(P.dn), tkw(P.tk_w);
  float ss = 0.f;
  const int i = threadIdx.x;
  if (i < CB) {
    const int c = cb * CB + i;
    // every load in flight before the sums (fixed order: groups, then ranks)
    float av[MK_MAX_KVH], wv[MK_MAX_TOPK], yv[MK_MAX_TOPK];
#pragma unroll
    for (int g = 0; g < MK_MAX_KVH; ++g) av[g] = g < P.KVH ? ao.ldf(g * H + c) : 0.f;
#pragma unroll
    for (int j = 0; j < MK_MAX_TOPK; ++j) {
      wv[j] = j < K ? tkw.ldf(j) : 0.f;
      yv[j] = j < K ? dn.ldf(j * H + c) : 0.f;
    }
    float h0;
    if (l == 0) {
      const int tok = P.tokens[0];
      h0 = (tok >= 0 && tok < P.V) ? bf2f(P.emb[(size_t)tok * H + c]) : 0.f;
    } else {
      h0 = h.ldf(c);
    }
    float a = 0.f;
#pragma unroll
    for (int g = 0; g < MK_MAX_KVH; ++g)
      if (g < P.KVH) a += av[g];
    float y = 0.f;
#pragma unroll
    for (int j = 0; j < MK_MAX_TOPK; ++j)
      if (j < K) y = fmaf(wv[j], yv[j], y);
    const float v = (h0 + a) + y;
    h.stf(c, v);
    ss = v * v;
  }
  ss = wave_sum(ss);
  if (lane_id() == 0) sm.vred[wave_id()] = ss;
  __syncthreads();
  if (threadIdx.x == 0) {
    float tot = 0.f;
    for (int k = 0; k < MK_WAVES; ++k) tot += sm.vred[k];
    Pub(P.ssq).stf(cb, tot);
  }
}

// After a contribution to column block cb: the last of the block's
// KVH + n_active contributions does the residual and signals the next layer.
__device__ void block_arrive(const mk_params& P, const mk_task& t, int ctr_base, int cb, Smem& sm) {
  const int n_active = __builtin_amdgcn_readfirstlane(Pub(P.route).ldi(0));
  const int old = arrive(P, ctr_base + cb, sm);
  if (old == P.KVH + n_active - 1) {
    residual_block(P, t.layer, cb, sm);
    arrive_nr(P, t.sig_ctr[0]);
  }
}

// ------------------------------------------------------------------ O proj
// O projection split-K by kv group: group g's heads contribute their slice
// of the K dimension as soon as that group's attention lands (megakernel
// post, section "Drop false dependencies"); one task per (group, column block).
template <int NCH>
__device__ __forceinline__ void op_oproj(const mk_params& P, const mk_task& t, Smem& sm) {
  const int l = t.layer, g = t.a[0], cb = t.a[1];
  const int DP = P.CB / 16, p0 = cb * DP;
  const int kc = P.QH * P.D / 32;
  const int c0 = g * P.G * P.D / 32, c1 = c0 + P.G * P.D / 32;
  const size_t pstride = (size_t)kc * 512;
  WTile<4, NCH> w;
  wtile_load(w, P.wo + l * P.s_wo + (size_t)p0 * pstride, pstride, DP, c0, c1);
  if (!wait_task(P, t, sm)) return;
  mark(sm, 0);
  gemv_b1(w, P.o + (size_t)g * P.G * P.D, DP, c0, c1, sm);
  mark(sm, 1);
  if (threadIdx.x < DP * 16) Pub(P.ao + (size_t)g * P.H).stf(p0 * 16 + threadIdx.x, sm.out[threadIdx.x]);
  block_arrive(P, t, t.a[2], cb, sm);
}

// ------------------------------------------------------------------ router
// Router logits over a K range of a panel range (partial sums); the task that
// completes the router does ROUTER_TOPK + ROUTE_FINALIZE (megakernel post,
// section "Tasks"): sum the partials in fixed order, top-k (ties to the lower
// expert index), softmax over the kept logits, the expert work queue.
__device__ void topk_finalize(const mk_params& P, int l, Smem& sm);

template <int NCH>
__device__ __forceinline__ void op_router(const mk_params& P, const mk_task& t, Smem& sm) {
  const int l = t.layer, p0 = t.a[0], np = t.a[1], c0 = t.a[2], c1 = t.a[3], ks = t.a[4];
  const int kc = P.H / 32;
  const size_t pstride = (size_t)kc * 512;
  WTile<2, NCH> w;
  wtile_load(w, P.wr + l * P.s_wr + (size_t)p0 * pstride, pstride, np, c0, c1);
  if (!wait_task(P, t, sm)) return;
  load_xhat(P, l, sm);
  mark(sm, 0);
  gemv_lds(w, sm.xc, np, c0, c1, sm);
  mark(sm, 1);
  const int n = p0 * 16 + threadIdx.x;
  if (threadIdx.x < np * 16 && n < P.E) Pub(P.rp + (size_t)ks * P.E).stf(n, sm.out[threadIdx.x]);
  const int old = arrive(P, t.a[5], sm);
  if (old == P.n_router_tasks - 1) {
    mark(sm, 2);
    topk_finalize(P, l, sm);
    mark(sm, 3);
    arrive_nr(P, t.sig_ctr[0]);
  }
}

// Top-k by ranking: expert i's rank is the number of experts ahead of it
// (a larger logit, or an equal logit and a lower index); the experts ranked
// below k are kept, in rank order. Every comparison is independent, so this
// runs in a few hundred cycles instead of k dependent rounds of a wave argmax.
__device__ void topk_finalize(const mk_params& P, int l, Smem& sm) {
  const int E = P.E, K = P.K;
  const int i = threadIdx.x;
  const Pub R(P.rp), TI(P.tk_idx), TW(P.tk_w), RT(P.route);
  float* lg = sm.u.tk.logit;
  if (i < E) {
    float p[MK_MAX_RKS];
#pragma unroll
    for (int k = 0; k < MK_MAX_RKS; ++k) p[k] = k < P.router_ks ? R.ldf(k * E + i) : 0.f;
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < MK_MAX_RKS; ++k)
      if (k < P.router_ks) v += p[k];
    lg[i] = v;
  }
  __syncthreads();
  if (i < E) {
    const float v = lg[i];
    int rank = 0;
    for (int j = 0; j < E; j += 4) {
      const float4 q = *(const float4*)(lg + j);
      rank += (q.x > v) | ((q.x == v) & (j + 0 < i));
      rank += (q.y > v) | ((q.y == v) & (j + 1 < i));
      rank += (q.z > v) | ((q.z == v) & (j + 2 < i));
      rank += (q.w > v) | ((q.w == v) & (j + 3 < i));
    }
    if (rank < K) {
      sm.u.tk.sel_idx[rank] = i;
      sm.u.tk.sel_val[rank] = v;
    }
  }
  __syncthreads();
  if (i < K) {
    // softmax over the kept logits (max-subtracted; rank 0 is the max),
    // summed in rank order
    const float top = sm.u.tk.sel_val[0];
    float sum = 0.f;
    for (int j = 0; j < K; ++j) sum += __expf(sm.u.tk.sel_val[j] - top);
    const int my_idx = sm.u.tk.sel_idx[i];
    const float ej = __expf(sm.u.tk.sel_val[i] - top);
    // batch 1: the k distinct experts are the active ones; queue them in
    // ascending expert order, with the token's slot j routed to each
    int pos = 0;
    for (int j = 0; j < K; ++j) pos += sm.u.tk.sel_idx[j] < my_idx;
    TI.sti(i, my_idx);
    TW.stf(i, ej / sum);
    RT.sti(4 + pos, my_idx);
    RT.sti(4 + E + pos, 1);
    RT.sti(4 + 2 * E + pos * P.B, i);
    if (P.tk_trace) P.tk_trace[(size_t)l * K + i] = my_idx;
    if (i == 0) {
      RT.sti(0, K);
      RT.sti(1, K * P.up_items_per_expert);
      RT.sti(2, K * P.down_items_per_expert);
    }
  }
}

__device__ __forceinline__ int claim(const mk_params& P, int32_t c, Smem& sm) {
  if (threadIdx.x == 0)
    sm.claim = (int)__hip_atomic_fetch_add(&P.ctr[c], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int id = sm.claim;
  __syncthreads();
  return id;
}

// Expert up/gate over one K half of one gate/up panel pair, claimed from the
// queue ROUTER_TOPK built (megakernel post, section "Tasks":
// MOE_UPGATE_ACT_DRAIN; the scheduler section of the Chinese version:
// claimers take the next entry atomically until the queue is empty). The two
// K halves' gate and up sums are added, and the SiLU-and-multiply applied,
// by the down projection that consumes them.
// Route entries of the layer's active experts into LDS (one round trip).
__device__ __forceinline__ void load_route(const mk_params& P, Smem& sm) {
  const Pub R(P.route);
  const int E = P.E;
  const int i = threadIdx.x;
  if (i < 4) sm.rt_hdr[i] = R.ldi(i);
  if (i < E) {
    sm.rt_e[i] = R.ldi(4 + i);
    sm.rt_slot[i] = R.ldi(4 + 2 * E + i * P.B);
  }
  __syncthreads();
}

// Claim n consecutive items of a work queue: returns (block-uniform) the first.
__device__ __forceinline__ int claim_n(const mk_params& P, int32_t c, int n, Smem& sm) {
  if (threadIdx.x == 0)
    sm.claim = (int)__hip_atomic_fetch_add(&P.ctr[c], (uint32_t)n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int id = sm.claim;
  __syncthreads();
  return id;
}

#define MK_UP_BATCH 4  // at most this many up/gate items claimed together, their weights in flight together

template <int NCH>
__device__ __forceinline__ void op_moe_up(const mk_params& P, const mk_task& t, Smem& sm) {
  if (!wait_task(P, t, sm)) return;
  const int l = t.layer, claim_ctr = t.a[0], done_base = t.a[1];
  const int F = P.F, upe = P.up_items_per_expert;
  const int kc = P.H / 32, kh_chunks = kc / 2;
  const size_t pstride = (size_t)kc * 512;
  const Pub GU(P.gu);
  load_route(P, sm);
  const int n_items = __builtin_amdgcn_readfirstlane(sm.rt_hdr[1]);
  // batch size: the queue spread over the claimers expected to be free
  const int nb = min(MK_UP_BATCH, max(1, (n_items + t.a[2] - 1) / t.a[2]));
  int id0 = claim_n(P, claim_ctr, nb, sm);
  load_xhat(P, l, sm);
  mark(sm, 0);
  bool first = true;
  while (id0 < n_items) {
    if (ld_relaxed(&P.err[0]) != 0) return;
    WTile<2, NCH> w[MK_UP_BATCH];
#pragma unroll
    for (int k = 0; k < MK_UP_BATCH; ++k) {
      const int id = id0 + k;
      const int a = id / upe, r = id % upe;
      const int tt = r >> 1, kh = r & 1;
      const int e = __builtin_amdgcn_readfirstlane(sm.rt_e[min(a, P.E - 1)]);
      const int c0 = kh * kh_chunks;
      // an item past the queue's end loads nothing (np = 0: a zero tile)
      wtile_load(w[k], P.wgu + l * P.s_wgu_l + (size_t)e * P.s_wgu_e + (size_t)(2 * tt) * pstride, pstride,
                 (k < nb && id < n_items) ? 2 : 0, c0, c0 + kh_chunks);
    }
    mark(sm, 1);
    // the next claim travels while the weights stream
    const int next = claim_n(P, claim_ctr, nb, sm);
#pragma unroll
    for (int k = 0; k < MK_UP_BATCH; ++k) {
      const int id = id0 + k;
      if (k >= nb || id >= n_items) break;
      const int a = id / upe, r = id % upe;
      const int tt = r >> 1, kh = r & 1;
      const int c0 = kh * kh_chunks;
      const int slot = __builtin_amdgcn_readfirstlane(sm.rt_slot[a]);
      gemv_lds(w[k], sm.xc, 2, c0, c0 + kh_chunks, sm);
      if (k == 0 && first) mark(sm, 2);
      // gu[slot][kh][gate|up][F]
      if (threadIdx.x < 32) {
        const int which = threadIdx.x >> 4, col = tt * 16 + (threadIdx.x & 15);
        GU.stf(((slot * 2 + kh) * 2 + which) * F + col, sm.out[threadIdx.x]);
      }
    }
    // one drain for the batch, then each item's arrival on its expert's counter
    sync_published();
    if ((int)threadIdx.x < nb && id0 + (int)threadIdx.x < n_items)
      __hip_atomic_fetch_add(&P.ctr[done_base + (id0 + (int)threadIdx.x) / upe], 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    if (first) mark(sm, 3);
    first = false;
    id0 = next;
  }
}

// Expert down over one column block, claiming (expert, block) items. Its
// weights stream before waiting for that expert's up/gate items (megakernel
// post, section "What we have done differently": MoE down streams weights
// while up/gate still computes the hidden state it consumes).
template <int NCH>
__device__ __forceinline__ void op_moe_down(const mk_params& P, const mk_task& t, Smem& sm) {
  if (!wait_task(P, t, sm)) return;
  const int l = t.layer, claim_ctr = t.a[0], done_base = t.a[1], blk_base = t.a[2];
  const int E = P.E, F = P.F, H = P.H;
  const int kc = F / 32;
  const size_t pstride = (size_t)kc * 512;
  const int DP = P.CB / 16;
  const Pub DN(P.dn), GU(P.gu);
  int id = claim(P, claim_ctr, sm);
  load_route(P, sm);
  const int n_items = __builtin_amdgcn_readfirstlane(sm.rt_hdr[2]);
  while (id < n_items) {
    if (ld_relaxed(&P.err[0]) != 0) return;
    const int a = id / P.down_items_per_expert, cb = id % P.down_items_per_expert;
    const int e = __builtin_amdgcn_readfirstlane(sm.rt_e[a]);
    WTile<4, NCH> w;
    wtile_load(w, P.wd + l * P.s_wd_l + (size_t)e * P.s_wd_e + (size_t)(cb * DP) * pstride, pstride, DP, 0, kc);
    // the next claim travels while the weights stream
    const int next = claim(P, claim_ctr, sm);
    if (!wait_one(P, done_base + a, P.up_items_per_expert, sm)) return;
    const int slot = __builtin_amdgcn_readfirstlane(sm.rt_slot[a]);
    // u = silu(g0 + g1) * (u0 + u1) over F, staged in LDS
    float* us = sm.us;
#pragma unroll
    for (int k = threadIdx.x; k < MK_MAX_F; k += MK_WG_THREADS) {
      if (k >= F) break;
      const float g0 = GU.ldf(((slot * 2 + 0) * 2 + 0) * F + k), g1 = GU.ldf(((slot * 2 + 1) * 2 + 0) * F + k);
      const float u0 = GU.ldf(((slot * 2 + 0) * 2 + 1) * F + k), u1 = GU.ldf(((slot * 2 + 1) * 2 + 1) * F + k);
      const float gt = g0 + g1;
      us[k] = gt / (1.0f + __expf(-gt)) * (u0 + u1);
    }
    __syncthreads();
    gemv_lds(w, us, DP, 0, kc, sm);
    if (threadIdx.x < DP * 16) DN.stf(slot * H + cb * DP * 16 + threadIdx.x, sm.out[threadIdx.x]);
    block_arrive(P, t, blk_base, cb, sm);
    id = next;
  }
}

// ----------------------------------------------------------------- LM head
// LM head panels with each task's argmax candidate; the task that completes
// the head picks the greedy token: the largest logit, the lowest index on
// ties (tiny-vllm walkthrough, section "The remaining layers and logits").
__device__ void final_argmax(const mk_params& P, Smem& sm);

template <int NCH>
__device__ __forceinline__ void op_lmhead(const mk_params& P, const mk_task& t, Smem& sm) {
  const int p0 = t.a[0], np = t.a[1], ord = t.a[2];
  const int kc = P.H / 32;
  const size_t pstride = (size_t)kc * 512;
  WTile<2, NCH> w;
  wtile_load(w, P.wlm + (size_t)p0 * pstride, pstride, np, 0, kc);
  if (!wait_task(P, t, sm)) return;
  load_xhat(P, P.L, sm);
  gemv_lds(w, sm.xc, np, 0, kc, sm);
  if (wave_id() == 0) {
    const int tid = threadIdx.x;
    float v = kNegInf;
    int ix = 0x7fffffff;
    if (tid < np * 16) {
      v = sm.out[tid];
      ix = p0 * 16 + tid;
      P.logits[ix] = v;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(v, o);
      const int oi = __shfl_xor(ix, o);
      if (ov > v || (ov == v && oi < ix)) { v = ov; ix = oi; }
    }
    if (tid == 0) {
      Pub(P.lm_val).stf(ord, v);
      Pub(P.lm_arg).sti(ord, ix);
    }
  }
  const int old = arrive(P, t.a[3], sm);
  if (old == P.n_lm_tasks - 1) final_argmax(P, sm);
}

__device__ void final_argmax(const mk_params& P, Smem& sm) {
  const int n = P.n_lm_tasks;
  const Pub LV(P.lm_val), LA(P.lm_arg);
  float v = kNegInf;
  int ix = 0x7fffffff;
  constexpr int U = 8;  // candidates per thread in flight together
  for (int base = 0; base < n; base += U * MK_WG_THREADS) {
    float cv[U];
    int ci[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * MK_WG_THREADS + threadIdx.x;
      cv[u] = i < n ? LV.ldf(i) : kNegInf;
      ci[u] = i < n ? LA.ldi(i) : 0x7fffffff;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (cv[u] > v || (cv[u] == v && ci[u] < ix)) { v = cv[u]; ix = ci[u]; }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(v, o);
    const int oi = __shfl_xor(ix, o);
    if (ov > v || (ov == v && oi < ix)) { v = ov; ix = oi; }
  }
  if (lane_id() == 0) {
    sm.vred[wave_id()] = v;
    sm.ired[wave_id()] = ix;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 0; k < MK_WAVES; ++k)
      if (sm.vred[k] > v || (sm.vred[k] == v && sm.ired[k] < ix)) { v = sm.vred[k]; ix = sm.ired[k]; }
    if (P.next_tokens) P.next_tokens[0] = ix;
    if (P.flags & 1u) {
      P.tokens[0] = ix;
      P.seq_lens[0] = P.seq_lens[0] + 1;
    }
  }
}

// --------------------------------------------------------------- dispatch

template <int D>
__device__ __forceinline__ void run_task(const mk_params& P, const mk_task& t, Smem& sm) {
  switch (t.op) {
    // chunks per wave: K / 32 / MK_WAVES for the largest K of each op
    // (hidden 2048, group width 1024, K half 1024, expert width 768)
    case MK_OP_QKV: op_qkv<64 / MK_WAVES>(P, t, sm); break;
    case MK_OP_ATTN: op_attn<D>(P, t, sm); break;
    case MK_OP_OPROJ: op_oproj<32 / MK_WAVES>(P, t, sm); break;
    case MK_OP_ROUTER: op_router<32 / MK_WAVES>(P, t, sm); break;
    case MK_OP_MOE_UP: op_moe_up<32 / MK_WAVES>(P, t, sm); break;
    case MK_OP_MOE_DOWN: op_moe_down<24 / MK_WAVES>(P, t, sm); break;
    case MK_OP_LMHEAD: op_lmhead<64 / MK_WAVES>(P, t, sm); break;
    default: wait_task(P, t, sm); break;
  }
}

}  // namespace

// The interpreter: workgroup i runs tasks [task_off[i], task_off[i+1]).
template <int D>
__global__ __launch_bounds__(MK_WG_THREADS, MK_WGS_PER_CU) void mk_interp(mk_params Pk) {
  __shared__ Smem sm;
  const mk_params& P = Pk;
  if (threadIdx.x == 0) {
    sm.xc_layer = -1;
    sm.t_mark[0] = sm.t_mark[1] = sm.t_mark[2] = sm.t_mark[3] = 0;
  }
  if (P.ctr_clear) {
    for (int i = blockIdx.x * MK_WG_THREADS + threadIdx.x; i < P.n_ctr; i += gridDim.x * MK_WG_THREADS)
      P.ctr_clear[i] = 0u;
  }
  __syncthreads();
  const int beg = P.task_off[blockIdx.x], end = P.task_off[blockIdx.x + 1];
  for (int i = beg; i < end; ++i) {
    const mk_task& t = P.tasks[i];
    const uint32_t t0 = (uint32_t)__builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) sm.t_mark[0] = sm.t_mark[1] = sm.t_mark[2] = sm.t_mark[3] = 0;
    run_task<D>(P, t, sm);
    __syncthreads();
    if (P.trace && threadIdx.x == 0) {
      // per-task timestamps (100 MHz device clock): start, waits satisfied,
      // inputs ready, computed, end
      uint32_t* rec = P.trace + (size_t)(P.trace_base + i) * 8;
      rec[0] = (uint32_t)t.op | ((uint32_t)t.layer << 8) | ((uint32_t)blockIdx.x << 16);
      rec[1] = t0;
      rec[2] = sm.t_waited;
      rec[3] = sm.t_mark[0];
      rec[4] = sm.t_mark[1];
      rec[5] = (uint32_t)__builtin_amdgcn_s_memrealtime();
      rec[6] = sm.t_mark[2];
      rec[7] = sm.t_mark[3];
    }
  }
}

template __global__ void mk_interp<64>(mk_params);
template __global__ void mk_interp<128>(mk_params);

// ------------------------------------------------------------- repacking
// Canonical row-major [K x N] (leading dimension ld) -> panel-tiled layout,
// source panel j written to destination panel dst0 + j*dstep. One workgroup
// per (32-row chunk, 512-column block, batch index z); z strides both sides.
extern "C" __global__ __launch_bounds__(256) void mk_repack_panels(const uint16_t* src, uint16_t* dst,
                                                                   int K, int N, int ld, int dst0, int dstep,
                                                                   size_t src_zstride, size_t dst_zstride) {
  __shared__ uint16_t tile[32][512 + 8];
  const int c = blockIdx.x;           // chunk row
  const int n0 = blockIdx.y * 512;    // first column
  const int z = blockIdx.z;
  const int width = min(512, N - n0);
  const uint16_t* s = src + z * src_zstride;
  uint16_t* d = dst + z * dst_zstride;
  const int kc = K / 32;
  for (int idx = threadIdx.x; idx < 32 * (width / 8); idx += 256) {
    const int row = idx / (width / 8), c8 = idx % (width / 8);
    const uint4 v = *(const uint4*)(s + (size_t)(32 * c + row) * ld + n0 + c8 * 8);
    *(uint4*)&tile[row][c8 * 8] = v;
  }
  __syncthreads();
  const int npan = width / 16;
  for (int idx = threadIdx.x; idx < npan * 64; idx += 256) {
    const int j = idx / 64, l = idx % 64;
    uint16_t tmp[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) tmp[i] = tile[8 * (l >> 4) + i][16 * j + (l & 15)];
    const int pj = dst0 + (n0 / 16 + j) * dstep;
    *(uint4*)(d + ((size_t)pj * kc + c) * 512 + l * 8) = *(uint4*)tmp;
  }
}

// ------------------------------------------------------------ host launch
#include "mk_launch.h"

hipError_t mk_launch_interp(const mk_params& P, int head_dim, int grid, bool cooperative, hipStream_t stream) {
  const void* fn = head_dim == 64 ? (const void*)mk_interp<64> : (const void*)mk_interp<128>;
  void* args[] = {(void*)&P};
  if (cooperative)
    return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(MK_WG_THREADS), args, 0, stream);
  return hipLaunchKernel(fn, dim3(grid), dim3(MK_WG_THREADS), args, 0, stream);
}

hipError_t mk_launch_repack(const uint16_t* src, uint16_t* dst, int K, int N, int ld, int dst0, int dstep,
                            int nz, size_t src_zstride, size_t dst_zstride, hipStream_t stream) {
  dim3 grid(K / 32, (N + 511) / 512, nz);
  hipLaunchKernelGGL(mk_repack_panels, grid, dim3(256), 0, stream, src, dst, K, N, ld, dst0, dstep, src_zstride,
                     dst_zstride);
  return hipGetLastError();
}

hipError_t mk_interp_occupancy(int head_dim, int* blocks_per_cu) {
  const void* fn = head_dim == 64 ? (const void*)mk_interp<64> : (const void*)mk_interp<128>;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, MK_WG_THREADS, 0);
}
