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
// the other XCDs' L2s (plain loads on one XCD were measured to return values
// another XCD had overwritten, within a launch and across launches). A C++
// release/acquire at agent scope is implemented by writing back / invalidating
// the whole L2 (buffer_wbl2 / buffer_inv), which costs microseconds per task,
// so the interpreter does not use them. Instead every activation that crosses
// compute units within a step is stored and loaded with device-scope (sc1)
// buffer instructions, which bypass the non-coherent cache levels; a producer
// waits for its own stores to complete (s_waitcnt) before its counter
// increment, and a consumer issues its loads only after it has observed the
// counter. Weights and the KV cache written in earlier steps are read with
// ordinary (non-temporal) loads: nothing writes them during a step, and kernel
// boundaries make earlier steps' writes visible to ordinary loads of data no
// XCD has cached (weights are never written after loading; a KV slot is
// written once, by the step that appends it, and read by later steps).
//
// Matrix products. Every projection runs on the matrix cores with the tokens
// as MFMA rows (16 per tile, batch <= 32 in two tiles) and 16 weight columns
// per panel: v_mfma_f32_16x16x32_bf16 takes the activations as the A operand
// (bf16) and one 1 KB chunk of a weight panel as the B operand, in exactly the
// layout the panels are stored in. The K dimension is spread over the 8 waves
// and their partial tiles are summed through LDS in a fixed order.
//
// Precision. A bf16 operand carries 8 significant bits; rounding every
// activation to it would add about 2^-9 relative error per projection and
// layer, which over 48 layers exceeds the float32 reference's tolerance. So
// every activation operand is a split pair: hi = bf16(x), lo = bf16(x - hi),
// and each product is two MFMAs (W hi + W lo), leaving about 2^-17 relative
// error; the weights and the KV cache are bf16 exactly as stored.
//
// Layer inputs. The residual add of a column block (the last contribution to
// arrive performs it) also writes u = bf16(h * gamma_next) and the block's
// per-token sum of squares. A consumer multiplies its projection of u by
// 1/sqrt(mean(h^2) + eps) per token, which equals projecting the RMS-normalised
// input (the norm's scale is a per-row factor), so no workgroup ever forms the
// normalised vector itself.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "mk_internal.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

namespace {

// ------------------------------------------------------------------ helpers

// The lane from mbcnt rather than from the work-item id: it depends on no
// register, so the compiler recomputes lane-derived values where it needs
// them instead of keeping the id live through the kernel and spilling it
// (a spill reload is a vector memory load, and waiting for it waits for
// every weight load issued before it).
__device__ __forceinline__ int lane_id() { return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }
// Wave index as a scalar (wave-uniform) value, so per-wave chunk choices
// compile to scalar branches instead of exec-mask juggling.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
// The thread's index in the workgroup, from the two above.
__device__ __forceinline__ int tid() { return (wave_id() << 6) | lane_id(); }

// The value of lane (this lane ^ M), M < 16, through ds_swizzle, whose
// pattern is an immediate: no per-lane address register (the compiler hoists
// lane-derived addresses out of the task loop and keeps them live through
// every op, as it does for ds_bpermute's).
template <int M>
__device__ __forceinline__ int xor_lane(int v) {
  static_assert(M > 0 && M < 16 && (M & (M - 1)) == 0, "power-of-two lane mask below 16");
  return __builtin_amdgcn_ds_swizzle(v, (M << 10) | 0x1f);
}
template <int M>
__device__ __forceinline__ float xor_lane(float v) {
  return __int_as_float(xor_lane<M>(__float_as_int(v)));
}
// The values of lanes (l, l ^ 16) and of lanes (l, l ^ 32), in lane order,
// from gfx950's VALU lane swaps (no LDS round trip): permlane16_swap of x
// with itself gives x[l & ~16] and x[l | 16]; permlane32_swap gives
// x[l & 31] and x[(l & 31) + 32]. Both lanes of a pair get the same two
// values in the same order, so any combination of them is identical in both.
__device__ __forceinline__ void pair16(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair32(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair16(int v, int& a, int& b) {
  const auto r = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
  a = (int)r[0];
  b = (int)r[1];
}
__device__ __forceinline__ void pair32(int v, int& a, int& b) {
  const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  a = (int)r[0];
  b = (int)r[1];
}
__device__ __forceinline__ float sum16(float v) {
  float a, b;
  pair16(v, a, b);
  return a + b;
}
__device__ __forceinline__ float sum32(float v) {
  float a, b;
  pair32(v, a, b);
  return a + b;
}
__device__ __forceinline__ float max16(float v) {
  float a, b;
  pair16(v, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float max32(float v) {
  float a, b;
  pair32(v, a, b);
  return fmaxf(a, b);
}
// Sum over aligned groups of n lanes (n a power of two, at most 64; every
// lane of a group ends with its sum), butterfly order.
__device__ __forceinline__ float group_sum(float v, int n) {
  if (n > 1) v += xor_lane<1>(v);
  if (n > 2) v += xor_lane<2>(v);
  if (n > 4) v += xor_lane<4>(v);
  if (n > 8) v += xor_lane<8>(v);
  if (n > 16) v = sum16(v);
  if (n > 32) v = sum32(v);
  return v;
}
// Sum over the lanes of a wave that share the lane bits below m (m a power
// of two, at most 32): lanes l, l ^ m, l ^ 2m, ...
__device__ __forceinline__ float group_sum_above(float v, int m) {
  if (m <= 1) v += xor_lane<1>(v);
  if (m <= 2) v += xor_lane<2>(v);
  if (m <= 4) v += xor_lane<4>(v);
  if (m <= 8) v += xor_lane<8>(v);
  if (m <= 16) v = sum16(v);
  if (m <= 32) v = sum32(v);
  return v;
}

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
// float -> bf16 bits, round to nearest even
__device__ __forceinline__ uint32_t f2bf(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) { return f2bf(a) | (f2bf(b) << 16); }
// The split pair of x: hi = bf16(x), lo = bf16(x - hi).
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  const uint32_t h = f2bf(x);
  hi = (uint16_t)h;
  lo = (uint16_t)f2bf(x - bf2f((uint16_t)h));
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
constexpr int kNT = 2;    // cache-policy bit: non-temporal (streamed once)

// Device-coherent access to a buffer shared across compute units.
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
  __device__ __forceinline__ void st16x4(int i, u32x2_t v) const {  // 4 bf16 at 16-bit index i (8-byte aligned)
    __builtin_amdgcn_raw_buffer_store_b64(v, r, i * 2, 0, kSC1);
  }
  __device__ __forceinline__ u32x4_t ld16x8(int i) const {  // 8 bf16 at 16-bit index i
    return __builtin_amdgcn_raw_buffer_load_b128(r, i * 2, 0, kSC1);
  }
  __device__ __forceinline__ u32x2_t ld16x4(int i) const {  // 4 bf16 at 16-bit index i
    return __builtin_amdgcn_raw_buffer_load_b64(r, i * 2, 0, kSC1);
  }
  // Tagged words (8 bytes: the value's 32 bits, then the tag), index i in words.
  __device__ __forceinline__ void st_tagged(int i, uint32_t v, uint32_t tag) const {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{v, tag}, r, i * 8, 0, kSC1);
  }
  __device__ __forceinline__ u32x4_t ld_tagged2(int i) const {  // words i, i + 1 (i even)
    return __builtin_amdgcn_raw_buffer_load_b128(r, i * 8, 0, kSC1);
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

// Workgroup barrier ordering LDS only. __syncthreads() also releases global
// memory: it waits for this wave's earlier global stores, and since the
// memory counter retires in order, for every load issued before them, which
// empties a pipeline of weight loads at each barrier. Used where the barrier
// separates LDS writes from LDS reads; hand-offs through global memory keep
// the draining forms (sync_published, the counter waits).
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

constexpr float kNegInf = -__builtin_inff();

// ------------------------------------------------------------------ LDS

struct SmemAttn {
  float m[MK_WAVES][16];
  float l[MK_WAVES][16];
  float o[MK_WAVES][128][17];
};

// Attention combine scratch: per split and head, the rescale factor and sum.
#define MK_MAX_SPLITS 256
struct SmemComb {
  float f[MK_MAX_SPLITS][16];
  float l[MK_MAX_SPLITS][16];
  float M[16];
  float L[16];
  alignas(16) float4 part[MK_WG_THREADS];  // per thread partition: partial sums of 4 outputs
};

struct SmemTopk {
  alignas(16) uint64_t key[MK_MAX_BATCH][128];  // ordered (logit, -index) keys; 0 beyond E
  alignas(16) float logit[MK_MAX_BATCH][128];
  float sel_val[MK_MAX_BATCH][MK_MAX_TOPK];
  int sel_idx[MK_MAX_BATCH][MK_MAX_TOPK];
  uint32_t tokmask[128];  // tokens (bit b) routed to each expert
  int apos[128];          // each expert's position among the active experts
  uint64_t ballot[2];
};

// Partial output tiles of the 8 waves: [wave][panel][row tile][16 x 16].
#define MK_RED_TILES 8  // panels x row tiles of the largest product
union SmemU {
  float red[MK_WAVES * MK_RED_TILES * 256];
  SmemAttn at;
  SmemComb cb;
  SmemTopk tk;
};

// LDS per workgroup: one workgroup per compute unit (more than half of
// gfx950's 160 KB).
struct Smem {
  SmemU u;
  alignas(16) float out[MK_RED_TILES * 256];     // summed tiles [panel][row tile][16][16]
  alignas(16) uint16_t act[MK_MAX_BATCH * MK_MAX_F];  // expert hidden rows (bf16), down projection input
  alignas(16) float ssq[MK_MAX_BATCH * 64];      // per-token sums of squares per column block
  float inv_rms[MK_MAX_BATCH];
  float tkw[MK_MAX_BATCH * MK_MAX_TOPK];
  int row_off[MK_UP_BATCH_MAX][MK_MAX_BATCH];    // activation row offsets of the current items
  float vred[MK_WAVES];
  int ired[MK_WAVES];
  int flag;
  int errflag;            // thread 0's reading of the device error word, for every wave
  int claim;
  int claim2;
  int old;                // value an arrival counter held before this workgroup's increment
  int t_old[2];
  uint32_t t_waited;
  uint32_t t_mark[4];     // op-defined intermediate timestamps (e.g. inputs ready, computed)
  int rt_hdr[4];          // route header: n_active, up items, down items
  int rt_e[128];          // active experts, ascending
  int rt_cnt[128];        // tokens routed to each active expert
  int rt_slot[128 * MK_MAX_BATCH];  // per active expert: its routed slots b * k + j, ascending b
  int done_cnt[128];      // claiming MoE: up/gate items done per active expert, not yet counted
  int tb[MK_FUSED_B + 1];  // fused MoE residual: each token's range of (claimer, token) rows
};
static_assert(2 * MK_FUSED_B * 1024 <= MK_MAX_BATCH * MK_MAX_F, "merged attention operand fits");
static_assert(2 * MK_FUSED_B * MK_MAX_H + 2 * MK_FUSED_B * 16 <= MK_MAX_BATCH * MK_MAX_F,
              "fused MoE operands fit the expert hidden-row buffer");
static_assert(offsetof(Smem, out) % 16 == 0 && offsetof(Smem, act) % 16 == 0 && offsetof(Smem, ssq) % 16 == 0,
              "LDS vectors 16-byte aligned");

__device__ __noinline__ void raise_error_w(uint32_t* err, uint32_t code, uint32_t detail, uint32_t value) {
  uint32_t expected = 0;
  if (__hip_atomic_compare_exchange_strong(&err[0], &expected, code, __ATOMIC_RELAXED,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
    __hip_atomic_store(&err[1], detail, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&err[2], value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&err[3], (uint32_t)blockIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}
// (the parameter block is not passed to an out-of-line call: that would make
// the compiler copy it to scratch memory)
#define raise_error(P, code, detail, value) raise_error_w((P).err, (code), (detail), (value))

// Spin (thread 0) until ctr[c] >= tgt for each wait, or until another
// workgroup raised an error, or until the time limit. Block-uniform result.
// force: wait even in the kernel-per-op variant (for producers in the same launch).
__device__ __forceinline__ bool wait_counters(const mk_params& P, const int32_t* cs, const int32_t* ts, int n, Smem& sm,
                                              bool force = false) {
  if (tid() == 0) {
    const bool active = P.waits_enabled || force;
    // the first reading of every counter and the error word in one round trip
    uint32_t v[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) v[i] = (i < n && active && cs[i] >= 0) ? ld_relaxed(P.ctr + cs[i]) : 0xffffffffu;
    int ok = ld_relaxed(&P.err[0]) == 0;
    if (ok && active) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        if (i >= n || !ok || cs[i] < 0) continue;
        const uint32_t* c = P.ctr + cs[i];
        const uint32_t tgt = (uint32_t)ts[i];
        uint32_t spins = 0;
        for (uint32_t x = v[i]; x < tgt; x = ld_relaxed(c)) {
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
  // (LDS-only barriers: a wave does not wait here for its own outstanding
  // loads and stores, such as this task's weight prefetch or the previous
  // task's tagged stores; the data a task reads after its waits is read with
  // device-coherent loads issued after them)
  lds_sync();
  const bool ok = sm.flag != 0;
  lds_sync();
  return ok;
}

__device__ __forceinline__ bool wait_task(const mk_params& P, const mk_task& t, Smem& sm) {
  return wait_counters(P, t.wait_ctr, t.wait_tgt, 3, sm);
}

__device__ __forceinline__ bool wait_one(const mk_params& P, int32_t c, int32_t tgt, Smem& sm, bool force = false) {
  return wait_counters(P, &c, &tgt, 1, sm, force);
}

// The device error word as thread 0 reads it (other threads: 0). Issued
// before a streaming loop's next weight loads, so waiting for it later does
// not wait for them (the memory counter retires in order).
__device__ __forceinline__ uint32_t error_peek(const mk_params& P) {
  return tid() == 0 ? ld_relaxed(&P.err[0]) : 0u;
}

// Whether thread 0's reading e shows a device error, the same answer in every
// wave (through LDS): a loop that stops on it stops in every wave together, so
// the workgroup's barriers keep matching.
__device__ __forceinline__ bool error_seen(uint32_t e, Smem& sm) {
  if (tid() == 0) sm.errflag = (int)e;
  lds_sync();
  const bool r = sm.errflag != 0;
  lds_sync();
  return r;
}

__device__ __forceinline__ int layer_window(const mk_params& P, int l) {
  if (P.window == 0) return 0;
  return (l % P.full_every) == P.full_every - 1 ? 0 : P.window;
}

// ------------------------------------------------------ tagged hand-offs
// A producer stores each value with its step's and layer's tag in one 8-byte
// device-coherent word (a single store: a reader sees the old word or the new
// one, never half of each) and moves on without waiting for the store to be
// acknowledged; a consumer loads the words until every tag is the expected
// one. This replaces, for small hand-offs, the store drain, the counter
// increment, the counter poll and the data load that follows it by one
// device-coherent round trip.
__device__ __forceinline__ uint32_t step_tag(const mk_params& P, int l) { return P.tag_base | (uint32_t)(l + 1); }

// Poll words w, w + 1 (w even) of a tagged buffer until both carry `tag`;
// false on the time limit or another workgroup's error (each thread polls on
// its own; the caller combines the results).
__device__ __forceinline__ bool poll_tagged2(const Pub& src, int w, uint32_t tag, const mk_params& P, u32x4_t& v) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  uint32_t spins = 0;
  for (v = src.ld_tagged2(w); v[1] != tag || v[3] != tag; v = src.ld_tagged2(w)) {
    __builtin_amdgcn_s_sleep(1);
    if ((++spins & 63u) == 0) {
      if (ld_relaxed(&P.err[0]) != 0) return false;
      if ((int64_t)(__builtin_amdgcn_s_memrealtime() - t0) > P.timeout_ticks) {
        raise_error(P, MK_DEVERR_TIMEOUT, 0xffff0000u | (uint32_t)w, v[1]);
        return false;
      }
    }
  }
  return true;
}

__device__ __forceinline__ void mark(Smem& sm, int k) {
  if (tid() == 0) sm.t_mark[k] = (uint32_t)__builtin_amdgcn_s_memrealtime();
}

// ---------------------------------------------------------- arrivals
// Count one arrival on counter c once every wave's device-coherent stores
// have completed.
__device__ __forceinline__ void arrive_nr(const mk_params& P, int32_t c) {
  sync_published();
  if (tid() == 0 && c >= 0)
    __hip_atomic_fetch_add(&P.ctr[c], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The same, returning (block-uniform) the value the counter held before this
// arrival, so the last of a known number of arrivals can act on the result.
__device__ __forceinline__ int arrive(const mk_params& P, int32_t c, Smem& sm) {
  sync_published();
  if (tid() == 0)
    sm.old = (int)__hip_atomic_fetch_add(&P.ctr[c], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int old = sm.old;
  __syncthreads();
  return old;
}

// Claim n consecutive items of a work queue: returns (block-uniform) the first.
__device__ __forceinline__ int claim_n(const mk_params& P, int32_t c, int n, Smem& sm) {
  if (tid() == 0)
    sm.claim = (int)__hip_atomic_fetch_add(&P.ctr[c], (uint32_t)n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  lds_sync();
  const int id = sm.claim;
  lds_sync();
  return id;
}

// ------------------------------------------------------- scratch addressing
// Layer inputs alternate between two buffers by layer parity: u and the sums
// of squares of layer l are read while layer l's residual adds write those of
// layer l + 1.
// u is stored as the split pair: part 0 = bf16(x), part 1 = bf16(x - part 0).
__device__ __forceinline__ const uint16_t* u_of(const mk_params& P, int l, int part) {
  return P.u + ((size_t)(l & 1) * 2 + part) * P.B * P.H;
}
__device__ __forceinline__ uint16_t* u_of_w(const mk_params& P, int l, int part) {
  return P.u + ((size_t)(l & 1) * 2 + part) * P.B * P.H;
}
// The attention output, split the same way: [hi|lo][B][QH*D].
__device__ __forceinline__ uint16_t* o_of(const mk_params& P, int part) {
  return P.o + (size_t)part * P.B * P.QH * P.D;
}
// Routing scratch, one region per layer (a compute unit may still read a
// layer's route after the next layer's router has run):
// router partials [ks][B][E], top-k ids and weights [B][K], route.
__device__ __forceinline__ float* rp_of(const mk_params& P, int l) {
  return P.rp + (size_t)l * P.router_ks * P.B * P.E;
}
__device__ __forceinline__ int32_t* tki_of(const mk_params& P, int l) { return P.tk_idx + (size_t)l * P.B * P.K; }
__device__ __forceinline__ float* tkw_of(const mk_params& P, int l) { return P.tk_w + (size_t)l * P.B * P.K; }
__device__ __forceinline__ int32_t* route_of(const mk_params& P, int l) {
  return P.route + (size_t)l * MK_ROUTE_INTS(P.E, P.B);
}
__device__ __forceinline__ float* ssq_of(const mk_params& P, int l) {
  return P.ssq + (size_t)(l & 1) * P.B * P.NB;
}

// 1/sqrt(mean(h^2) + eps) of every token from the column blocks' sums of
// squares in sm.ssq ([B][NB], written before a barrier): 32 lanes per token,
// each summing every 32nd block, then a butterfly; into sm.inv_rms.
__device__ __forceinline__ void inv_rms_lds(const mk_params& P, Smem& sm) {
  const int NB = P.NB;
#pragma unroll
  for (int k = 0; k < MK_MAX_BATCH * 32 / MK_WG_THREADS; ++k) {
    // (waves whose tokens are all past the batch skip the exchange)
    if ((wave_id() * 64 + k * MK_WG_THREADS) / 32 < P.B) {
      const int i = tid() + k * MK_WG_THREADS, b = i >> 5, j = i & 31;
      float v = 0.f;
      if (b < P.B)
        for (int q = j; q < NB; q += 32) v += sm.ssq[b * NB + q];
      v = group_sum(v, 32);
      if (b < P.B && j == 0) sm.inv_rms[b] = 1.0f / sqrtf(v / (float)P.H + P.eps);
    }
  }
}

// The same for layer l's input, loading the sums of squares.
__device__ __forceinline__ void load_inv_rms(const mk_params& P, int l, Smem& sm) {
  const Pub S(ssq_of(P, l));
  const int n = P.B * P.NB;
  for (int i = tid(); i < n; i += MK_WG_THREADS) sm.ssq[i] = S.ldf(i);
  lds_sync();
  inv_rms_lds(P, sm);
  lds_sync();
}

// --------------------------------------------------------- matrix tiles
//
// Weight matrices [K x N] are stored panel-tiled: 16-column panels, each a run
// of K/32 chunks of 1 KB; in a chunk, lane l holds the 8 bf16 of rows
// 32c + 8(l/16) + i (i = 0..7) of column 16j + l%16 (the B operand of
// v_mfma_f32_16x16x32_bf16). Chunk c of a panel goes to wave c % 8, so every
// load is one contiguous 1 KB line per wave.
template <int NP, int NCH>
struct WTile {
  u32x4_t v[NP][NCH];
};

// Chunks outside [c0, c1) and panels at or beyond np are zero. The loads go
// through one buffer resource over the np panels, a chunk outside the range
// reading past its end (which returns zeros): no branches, so the compiler
// counts the loads in flight exactly and waits only for the ones it uses.
template <int NP, int NCH>
__device__ __forceinline__ void wtile_load(WTile<NP, NCH>& w, const uint16_t* base, size_t pstride,
                                           int np, int c0, int c1) {
  const int wv = wave_id(), ln = lane_id();
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, np * (int)pstride * 2, 0x00020000);
#pragma unroll
  for (int pp = 0; pp < NP; ++pp)
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = c0 + wv + MK_WAVES * i;
      const int off = (pp < np && c < c1) ? (pp * (int)pstride + c * 512) * 2 + ln * 16 : 0x7ffffff0;
      w.v[pp][i] = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNT);
    }
}

// Activation operand: MT row tiles of 16 tokens; lane l holds the 8 bf16 of
// row 16 mt + l%16 at K offsets 32c + 8(l/16) .. +7 of each of its chunks.
template <int MT, int NCH>
struct ATile {
  u32x4_t a[MT][NCH];
};

// A rows from a bf16 matrix shared across compute units; row r starts at
// element offset off[r] (negative: a zero row). Chunks are absolute: row
// element 32c + 8(l/16). Chunks outside [c0, c1) are zero.
template <int MT, int NCH>
__device__ __forceinline__ void atile_load_bf16(ATile<MT, NCH>& A, const Pub& src, const int* off, int c0, int c1) {
  const int wv = wave_id(), ln = lane_id();
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int o = off[mt * 16 + (ln & 15)];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = c0 + wv + MK_WAVES * i;
      A.a[mt][i] = (c < c1 && o >= 0) ? src.ld16x8(o + 32 * c + 8 * (ln >> 4)) : u32x4_t{0u, 0u, 0u, 0u};
    }
  }
}

// One row tile whose rows each lane names itself: o is the element offset of
// row l%16 (negative: a zero row). Otherwise as atile_load_bf16.
template <int NCH>
__device__ __forceinline__ void atile_load_row(ATile<1, NCH>& A, const Pub& src, int o, int c0, int c1) {
  const int wv = wave_id(), ln = lane_id();
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = c0 + wv + MK_WAVES * i;
    A.a[0][i] = (c < c1 && o >= 0) ? src.ld16x8(o + 32 * c + 8 * (ln >> 4)) : u32x4_t{0u, 0u, 0u, 0u};
  }
}

// A rows from a float32 matrix shared across compute units, rounded to bf16;
// row r starts at off[r]; chunk c reads row elements 32 (c - c0) + 8(l/16).
template <int MT, int NCH>
__device__ __forceinline__ void atile_load_f32(ATile<MT, NCH>& A, const Pub& src, const int* off, int c0, int c1) {
  const int wv = wave_id(), ln = lane_id();
  float4 x[MT][NCH][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int o = off[mt * 16 + (ln & 15)];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = c0 + wv + MK_WAVES * i;
      if (c < c1 && o >= 0) {
        const int e = o + 32 * (c - c0) + 8 * (ln >> 4);
        x[mt][i][0] = src.ldf4(e);
        x[mt][i][1] = src.ldf4(e + 4);
      } else {
        x[mt][i][0] = x[mt][i][1] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const float4 p = x[mt][i][0], q = x[mt][i][1];
      A.a[mt][i] = u32x4_t{pack_bf2(p.x, p.y), pack_bf2(p.z, p.w), pack_bf2(q.x, q.y), pack_bf2(q.z, q.w)};
    }
}

template <int NP, int MT>
struct Acc {
  f32x4_t c[NP][MT];
};

// acc = (A hi + A lo) W over this wave's chunks.
template <int NP, int MT, int NCH>
__device__ __forceinline__ void mfma_tiles(Acc<NP, MT>& acc, const WTile<NP, NCH>& w, const ATile<MT, NCH>& Ah,
                                           const ATile<MT, NCH>& Al) {
#pragma unroll
  for (int pp = 0; pp < NP; ++pp)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc.c[pp][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NCH; ++i)
#pragma unroll
    for (int pp = 0; pp < NP; ++pp)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc.c[pp][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, Al.a[mt][i]),
                                                                __builtin_bit_cast(bf16x8_t, w.v[pp][i]),
                                                                acc.c[pp][mt], 0, 0, 0);
        acc.c[pp][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, Ah.a[mt][i]),
                                                                __builtin_bit_cast(bf16x8_t, w.v[pp][i]),
                                                                acc.c[pp][mt], 0, 0, 0);
      }
}

// acc += (A hi + A lo) W over this wave's chunks.
template <int NP, int MT, int NCH>
__device__ __forceinline__ void mfma_tiles_add(Acc<NP, MT>& acc, const WTile<NP, NCH>& w, const ATile<MT, NCH>& Ah,
                                               const ATile<MT, NCH>& Al) {
#pragma unroll
  for (int i = 0; i < NCH; ++i)
#pragma unroll
    for (int pp = 0; pp < NP; ++pp)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc.c[pp][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, Al.a[mt][i]),
                                                                __builtin_bit_cast(bf16x8_t, w.v[pp][i]),
                                                                acc.c[pp][mt], 0, 0, 0);
        acc.c[pp][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, Ah.a[mt][i]),
                                                                __builtin_bit_cast(bf16x8_t, w.v[pp][i]),
                                                                acc.c[pp][mt], 0, 0, 0);
      }
}

// Sum the 8 waves' partial tiles (fixed order) into sm.out, indexed
// [(pp * MT + mt) * 256 + row * 16 + col].
template <int NP, int MT>
__device__ __forceinline__ void reduce_tiles(const Acc<NP, MT>& acc, Smem& sm) {
  static_assert(NP * MT <= MK_RED_TILES, "reduction buffer");
  constexpr int N = NP * MT * 256;
  const int wv = wave_id(), ln = lane_id();
  float* red = sm.u.red + wv * N;
#pragma unroll
  for (int pp = 0; pp < NP; ++pp)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[(pp * MT + mt) * 256 + (4 * (ln >> 4) + i) * 16 + (ln & 15)] = acc.c[pp][mt][i];
  lds_sync();
#pragma unroll
  for (int o = tid(); o < N; o += MK_WG_THREADS) {
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < MK_WAVES; ++k) s += sm.u.red[k * N + o];
    sm.out[o] = s;
  }
  lds_sync();
}

// ------------------------------------------------ FP8 feed-forward weights
// The post's roadmap names FP8 as the next, narrower weight type (Chinese
// version, section "下一步"). Codes are OCP E4M3 with one float32 scale per
// hidden unit for each of its gate column, up column and down row (code value
// times scale). Every E4M3 value is exactly a bf16 value, so the gate/up codes
// become the matrix cores' bf16 B operand in registers and the products run
// as for bf16 weights; the scales apply to the hidden unit's gate and up sums
// and, for the down row, to the unit's SiLU-and-multiply output.
//
// Gate/up panels: each 16-column panel is a run of K / 64 chunk pairs of
// 1 KB; in pair p, lane l holds 16 bytes: the codes of rows 64p + 8(l/16) + i
// (i = 0..7) of column l%16, then those of rows 64p + 32 + 8(l/16) + i. Pair
// p goes to wave p % 8: each load is one contiguous 1 KB line per wave.
template <int NP, int NPR>
struct WTile8 {
  u32x4_t v[NP][NPR];
};

// Pairs outside [p0, p1) and panels at or beyond np are zero (one buffer
// resource, out-of-range reads return zeros).
template <int NP, int NPR>
__device__ __forceinline__ void wtile8_load(WTile8<NP, NPR>& w, const uint8_t* base, int pstride, int np, int p0,
                                            int p1) {
  const int wv = wave_id(), ln = lane_id();
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, np * pstride, 0x00020000);
#pragma unroll
  for (int pp = 0; pp < NP; ++pp)
#pragma unroll
    for (int i = 0; i < NPR; ++i) {
      const int p = p0 + wv + MK_WAVES * i;
      const int off = (pp < np && p < p1) ? pp * pstride + p * 1024 + ln * 16 : 0x7ffffff0;
      w.v[pp][i] = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNT);
    }
}

// Four E4M3 codes -> their values as two words of bf16 pairs (codes 0, 1 in
// lo; 2, 3 in hi). The hardware conversion gives float32 values of at most
// four significant bits, so keeping their upper halves is exact.
__device__ __forceinline__ void e4m3x4_to_bf16(uint32_t c, uint32_t& lo, uint32_t& hi) {
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(c, false);
  const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(c, true);
  lo = __builtin_amdgcn_perm(__float_as_uint(a[1]), __float_as_uint(a[0]), 0x07060302u);
  hi = __builtin_amdgcn_perm(__float_as_uint(b[1]), __float_as_uint(b[0]), 0x07060302u);
}

// One lane's 16 codes of a chunk pair -> the bf16 B operands of its two chunks.
__device__ __forceinline__ void e4m3x16_to_bf16(const u32x4_t& c, u32x4_t& c0, u32x4_t& c1) {
  uint32_t w[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) e4m3x4_to_bf16(c[k], w[2 * k], w[2 * k + 1]);
  c0 = u32x4_t{w[0], w[1], w[2], w[3]};
  c1 = u32x4_t{w[4], w[5], w[6], w[7]};
}

// The activation operand matching a WTile8: slot 2i + h holds chunk
// 2 (p0 + wave + 8 i) + h of the layer input staged in LDS (zero past p1).
template <int NCH>
__device__ __forceinline__ void atile_lds_pairs(ATile<1, NCH>& A, const uint16_t* xs, int H, int B, int p0, int p1) {
  const int wv = wave_id(), ln = lane_id(), row = ln & 15;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int p = p0 + wv + MK_WAVES * (i / 2), c = 2 * p + (i % 2);
    A.a[0][i] = (p < p1 && row < B) ? *(const u32x4_t*)(xs + row * H + 32 * c + 8 * (ln >> 4)) : u32x4_t{0u, 0u, 0u, 0u};
  }
}

// acc (+)= (A hi + A lo) W over this wave's chunk pairs, W in E4M3 codes.
template <int NP, int NPR>
__device__ __forceinline__ void mfma_tiles8(Acc<NP, 1>& acc, const WTile8<NP, NPR>& w, const ATile<1, 2 * NPR>& Ah,
                                            const ATile<1, 2 * NPR>& Al, bool add) {
  if (!add) {
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) acc.c[pp][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int i = 0; i < NPR; ++i)
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      u32x4_t b[2];
      e4m3x16_to_bf16(w.v[pp][i], b[0], b[1]);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        acc.c[pp][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, Al.a[0][2 * i + h]),
                                                               __builtin_bit_cast(bf16x8_t, b[h]), acc.c[pp][0], 0, 0, 0);
        acc.c[pp][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, Ah.a[0][2 * i + h]),
                                                               __builtin_bit_cast(bf16x8_t, b[h]), acc.c[pp][0], 0, 0, 0);
      }
    }
}

// Down rows in E4M3: slice s (rows 16 s .. 16 s + 15) of an FFN's [F x H]
// down matrix is H runs of 16 bytes, run h holding the codes of rows
// 16 s .. 16 s + 15 of column h (one contiguous 16 H bytes per slice).
// Thread t takes columns t + 512 j. An invalid slice reads nothing (zeros).
template <int NJ8>
struct DTile8 {
  u32x4_t v[NJ8];
};

template <int NJ8>
__device__ __forceinline__ void dtile8_load(DTile8<NJ8>& d, const uint8_t* slice, int H, bool valid) {
  const int t = tid();
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(slice), (short)0, valid ? H * 16 : 0, 0x00020000);
#pragma unroll
  for (int j = 0; j < NJ8; ++j) {
    const int h = t + MK_WG_THREADS * j;
    d.v[j] = __builtin_amdgcn_raw_buffer_load_b128(r, h < H ? h * 16 : 0x7ffffff0, 0, kNT);
  }
}

// Row tile of one K half in the chunk-pair order of FP8 weights: slot 2i + h
// holds chunk 2 (p0 + wave + 8 i) + h of row o (negative: a zero row).
template <int NCH>
__device__ __forceinline__ void atile_load_row_pairs(ATile<1, NCH>& A, const Pub& src, int o, int p0, int p1) {
  const int wv = wave_id(), ln = lane_id();
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int p = p0 + wv + MK_WAVES * (i / 2), c = 2 * p + (i % 2);
    A.a[0][i] = (p < p1 && o >= 0) ? src.ld16x8(o + 32 * c + 8 * (ln >> 4)) : u32x4_t{0u, 0u, 0u, 0u};
  }
}

// Row offsets of the batch's tokens (row b at b * stride + base), -1 beyond.
__device__ __forceinline__ void set_rows_batch(const mk_params& P, Smem& sm, int slot, int stride, int base) {
  if (tid() < MK_MAX_BATCH) sm.row_off[slot][tid()] = (int)tid() < P.B ? (int)tid() * stride + base : -1;
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
// SB: splits in flight per thread and round; MLR: rounds of 512 (split, head)
// maxima and sums held in registers (the rest load straight into LDS).
template <int D, int SB = MK_COMB_SB, int MLR = MK_MAX_SPLITS * 16 / MK_WG_THREADS>
__device__ __forceinline__ void attn_combine(const mk_params& P, int b, int g, int ns, Smem& sm,
                                             uint16_t* lds_h = nullptr, uint16_t* lds_l = nullptr,
                                             bool to_global = true);

// One wave's operands of one KV page of one kv group: K rows (keys) for the
// score MFMA, V^T tiles for the output MFMA.
template <int D>
struct KVPage {
  u32x4_t k[D / 32];
  u32x2_t v[D / 16];
};

// Tagged hand-off from layer l's QKV tasks: the G query heads of kv group g
// of sequence b (G * D floats) and the group's new key and value (2 D bf16),
// polled as tagged words (each thread its own pairs) and placed in LDS: the
// queries at sm.act as floats, the key and value after the first 1024 floats.
__device__ __forceinline__ bool poll_qkv(const mk_params& P, int l, int b, int g, Smem& sm) {
  const uint32_t tag = step_tag(P, l);
  const int D = P.D, GD = P.G * D, nq = GD / 2, n = nq + D;
  float* qs = reinterpret_cast<float*>(sm.act);
  uint16_t* kvs = reinterpret_cast<uint16_t*>(qs + 1024);
  const Pub QT(P.qt + (size_t)b * P.QH * D + (size_t)g * GD), KT(P.kvt + (size_t)(b * P.KVH + g) * 2 * D);
  if (tid() == 0) sm.flag = 1;
  lds_sync();
  bool ok = true;
  for (int j = tid(); j < n && ok; j += MK_WG_THREADS) {
    u32x4_t v;
    if (j < nq) {
      ok = poll_tagged2(QT, 2 * j, tag, P, v);
      qs[2 * j] = __uint_as_float(v[0]);
      qs[2 * j + 1] = __uint_as_float(v[2]);
    } else {
      const int w = 2 * (j - nq);
      ok = poll_tagged2(KT, w, tag, P, v);
      kvs[w] = (uint16_t)v[0];
      kvs[w + 1] = (uint16_t)v[2];
    }
  }
  if (!ok) sm.flag = 0;
  lds_sync();
  const bool all = sm.flag != 0;
  if (tid() == 0) sm.t_waited = (uint32_t)__builtin_amdgcn_s_memrealtime();
  lds_sync();
  return all;
}

// One split (b, g, s): waits until the QKV tasks of group g are done
// (qkv_ctr >= qkv_tgt), counts itself on attn_ctr, and the last of the ns
// splits combines them and signals sig_ctr.
template <int D>
__device__ __forceinline__ void attn_split(const mk_params& P, int l, int b, int g, int s, int ns, int pps,
                                           int qkv_ctr, int qkv_tgt, int attn_ctr, int sig_ctr, bool merged_later,
                                           Smem& sm) {
  constexpr int NC = D / 32;
  constexpr int NT = D / 16;
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
  // With tagged hand-offs the new row comes from the tagged words instead
  // (patched in below), and the page's older rows, written by earlier steps,
  // stream before the wait like any other page.
  const bool tg = P.tagged != 0;
  const Pub KV(kvl);
  auto load_page = [&](int lp) {
    KVPage<D> pg;
    const int phys = P.bt[b * P.mpps + lp];
    if (phys < 0 || phys >= P.n_pages) {
      bad = true;
      return pg;
    }
    const int ko = ((phys * 2 + 0) * P.KVH + g) * (int)plane, vo = ((phys * 2 + 1) * P.KVH + g) * (int)plane;
    if (lp == lp_last && !tg) {
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
  const bool early0 = lp < my1 && (tg || lp != lp_last), early1 = lpn < my1 && (tg || lpn != lp_last);
  KVPage<D> cur, nxt;
  if (early0) cur = load_page(lp);
  if (early1) nxt = load_page(lpn);
  // the queries and the new key and value: the tagged words into LDS, or the
  // QKV tasks' counter
  float* qs = reinterpret_cast<float*>(sm.act);           // [G * D] queries
  const uint16_t* kn = reinterpret_cast<uint16_t*>(qs + 1024);  // [D] new key, then [D] new value
  if (tg) {
    if (!poll_qkv(P, l, b, g, sm)) return;
  } else if (!wait_one(P, qkv_ctr, qkv_tgt, sm)) {
    return;
  }
  if (!seq_ok) {
    if (tid() == 0) raise_error(P, MK_DEVERR_FAULT, 4000 + b, (uint32_t)seq);
    return;
  }
  if (lp < my1 && !early0) cur = load_page(lp);
  if (lpn < my1 && !early1) nxt = load_page(lpn);

  // Q^T operand (split pair): lane holds q[head ln%16][dims 32c + 8(ln/16) + i]
  bf16x8_t qb[NC], ql[NC];
  {
    const int hh = ln & 15;
    const Pub Q(P.q + (size_t)b * P.QH * D + (size_t)g * G * D);
    const int qo = min(hh, G - 1) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int e = qo + 32 * c + 8 * (ln >> 4);
      const float4 a0 = tg ? *(const float4*)(qs + e) : Q.ldf4(e), a1 = tg ? *(const float4*)(qs + e + 4) : Q.ldf4(e + 4);
      const float qv[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      u32x4_t pk, pl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint16_t h0, l0, h1, l1;
        split_bf16(qv[2 * i], h0, l0);
        split_bf16(qv[2 * i + 1], h1, l1);
        pk[i] = hh < G ? ((uint32_t)h0 | ((uint32_t)h1 << 16)) : 0u;
        pl[i] = hh < G ? ((uint32_t)l0 | ((uint32_t)l1 << 16)) : 0u;
      }
      qb[c] = __builtin_bit_cast(bf16x8_t, pk);
      ql[c] = __builtin_bit_cast(bf16x8_t, pl);
    }
  }

  f32x4_t oacc[NT];
#pragma unroll
  for (int d = 0; d < NT; ++d) oacc[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, lsum = 0.f;

  // online softmax over one page (keys as MFMA rows), positions [vlo, vhi]
  auto do_page = [&](const KVPage<D>& pg, int lp, int vlo, int vhi) {
    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, pg.k[c]), ql[c], sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, pg.k[c]), qb[c], sacc, 0, 0, 0);
    }
    float sv[4];
    float mloc = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pos = lp * PS + 4 * (ln >> 4) + i;
      sv[i] = (pos >= vlo && pos <= vhi) ? sacc[i] * scale : kNegInf;
      mloc = fmaxf(mloc, sv[i]);
    }
    mloc = max32(max16(mloc));
    const float mnew = fmaxf(m, mloc);
    if (mnew != kNegInf) {
      const float alpha = (m == kNegInf) ? 0.f : __expf(m - mnew);
      // the probabilities as a split pair too: with context values of mixed
      // sign the output is a near-cancelling average, and bf16 probabilities
      // alone would leave it about 2^-9 relative error at any length
      uint32_t ph[4], pl[4];
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = sv[i] == kNegInf ? 0.f : __expf(sv[i] - mnew);
        ph[i] = f2bf(pv);
        pl[i] = f2bf(pv - bf2f((uint16_t)ph[i]));
        ps += pv;
      }
      ps = sum32(sum16(ps));
      lsum = lsum * alpha + ps;
      m = mnew;
      const s16x4_t pH = {(short)ph[0], (short)ph[1], (short)ph[2], (short)ph[3]};
      const s16x4_t pL = {(short)pl[0], (short)pl[1], (short)pl[2], (short)pl[3]};
#pragma unroll
      for (int d = 0; d < NT; ++d) {
        oacc[d] *= alpha;
        oacc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, pg.v[d]), pL, oacc[d], 0, 0, 0);
        oacc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, pg.v[d]), pH, oacc[d], 0, 0, 0);
      }
    }
  };
  // two pages in registers: each wave computes one while the page two ahead
  // of it streams into the other's registers
  // (tagged: position p is left out of its page and taken from the tagged
  // words below)
  const int phi = tg ? p - 1 : p;
  while (lp < my1 && !bad) {
    do_page(cur, lp, lo, phi);
    if (lp + 2 * MK_WAVES < my1) cur = load_page(lp + 2 * MK_WAVES);
    lp += MK_WAVES;
    if (lp >= my1 || bad) break;
    do_page(nxt, lp, lo, phi);
    if (lp + 2 * MK_WAVES < my1) nxt = load_page(lp + 2 * MK_WAVES);
    lp += MK_WAVES;
  }
  if (bad) raise_error(P, MK_DEVERR_FAULT, 5000 + b, (uint32_t)lp);
  // tagged: the new token as a page of one key, on the wave that had its
  // page (key row p % PS of the K operand, element p % 4 of the V^T lanes
  // holding positions 4 (ln / 16) .. + 3)
  if (tg && !bad && lp_last >= my0 && lp_last < my1 && wv == (lp_last - my0) % MK_WAVES) {
    const int r = p % PS, e = r & 3;
    KVPage<D> vp;
    const bool krow = (ln & 15) == r, vq = (ln >> 4) == (r >> 2);
#pragma unroll
    for (int c = 0; c < NC; ++c)
      vp.k[c] = krow ? *(const u32x4_t*)(kn + 32 * c + 8 * (ln >> 4)) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int d = 0; d < NT; ++d) {
      const uint32_t v = vq ? (uint32_t)kn[D + 16 * d + (ln & 15)] : 0u;
      const uint32_t sh = (e & 1) ? (v << 16) : v;
      vp.v[d] = (e >> 1) ? u32x2_t{0u, sh} : u32x2_t{sh, 0u};
    }
    do_page(vp, lp_last, p, p);
  }

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
  for (int idx = tid(); idx < G * D; idx += MK_WG_THREADS) {
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
  if (merged_later) {  // the O projection tasks merge the splits
    arrive_nr(P, attn_ctr);
    return;
  }
  const int old = arrive(P, attn_ctr, sm);
  mark(sm, 1);
  if (old == ns - 1) {
    attn_combine<D>(P, b, g, ns, sm);
    mark(sm, 3);
    arrive_nr(P, sig_ctr);
  }
}

// Attention claimer (megakernel post, Chinese version, scheduler section:
// ATTN_DRAIN claimers steal the next split from the layer's shared queue
// until it is empty): items (b, g, s) in that order, so a split never waits
// behind a slow task on a particular compute unit.
//   a[0] claim counter, a[1] QKV counter base (per group), a[2] QKV tasks per
//   group, a[3] splits per (sequence, group), a[4] pages per split,
//   a[5] attention counter base (per sequence and group); sig_ctr[0]: the
//   combined-output counter base (per group).
template <int D>
__device__ __forceinline__ void op_attn(const mk_params& P, const mk_task& t, Smem& sm) {
  const int ns = t.a[3], n_items = P.B * P.KVH * ns;
  int id = claim_n(P, t.a[0], 1, sm);
  while (id < n_items) {
    const int bg = id / ns, s = id % ns, b = bg / P.KVH, g = bg % P.KVH;
    // b[0] = 1: the splits count per group (all sequences); the O projection merges them
    const bool ml = t.b[0] == 1;
    attn_split<D>(P, t.layer, b, g, s, ns, t.a[4], t.a[1] + g, t.a[2], t.a[5] + (ml ? g : bg), t.sig_ctr[0] + g, ml,
                  sm);
    if (error_seen(error_peek(P), sm)) return;
    id = claim_n(P, t.a[0], 1, sm);
  }
}

// Log-sum-exp merge of one (sequence, kv group)'s split partials into the
// attention output (megakernel post, section "Tasks": ATTN_COMBINE):
// o = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s, splits in fixed order.
template <int D, int SB, int MLR>
__device__ __forceinline__ void attn_combine(const mk_params& P, int b, int g, int ns, Smem& sm, uint16_t* lds_h,
                                             uint16_t* lds_l, bool to_global) {
  const int G = P.G;
  const int stride = G * D + 2 * G;
  const Pub src(P.part + (size_t)(b * P.KVH + g) * P.max_splits * stride);
  SmemComb& C = sm.u.cb;
  // 16-byte loads of the outputs: a split's G * D outputs are GD4 groups of
  // four; the workgroup forms NP partitions of GD4 threads, partition p
  // taking splits p, p + NP, ..., up to SB of them in flight at a time
  const int GD4 = G * D / 4, NP = MK_WG_THREADS / GD4;
  const int part = tid() / GD4, j = tid() % GD4, hh = 4 * j / D;
  // every split's maxima and sums and the first round of outputs: one round trip
  float mv[MLR], lv[MLR];
#pragma unroll
  for (int k = 0; k < MLR; ++k) {
    const int i = tid() + k * MK_WG_THREADS, s = i / G, h2 = i % G;
    mv[k] = i < ns * G ? src.ldf(s * stride + G * D + h2) : kNegInf;
    lv[k] = i < ns * G ? src.ldf(s * stride + G * D + G + h2) : 0.f;
  }
  float4 v[SB];
#pragma unroll
  for (int k = 0; k < SB; ++k) {
    const int s = part + k * NP;
    v[k] = (part < NP && s < ns) ? src.ldf4(s * stride + 4 * j) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int k = 0; k < MLR; ++k) {
    const int i = tid() + k * MK_WG_THREADS, s = i / G, h2 = i % G;
    if (i < ns * G) {
      C.f[s][h2] = mv[k];
      C.l[s][h2] = lv[k];
    }
  }
  for (int i = tid() + MLR * MK_WG_THREADS; i < ns * G; i += MK_WG_THREADS) {
    const int s = i / G, h2 = i % G;
    C.f[s][h2] = src.ldf(s * stride + G * D + h2);
    C.l[s][h2] = src.ldf(s * stride + G * D + G + h2);
  }
  __syncthreads();
  // per head (32 lanes each): the maximum over the splits
  {
    const int h2 = tid() >> 5, jj = tid() & 31;
    float M = kNegInf;
    if (h2 < G)
      for (int s = jj; s < ns; s += 32) M = fmaxf(M, C.f[s][h2]);
    M = fmaxf(M, xor_lane<1>(M));
    M = fmaxf(M, xor_lane<2>(M));
    M = fmaxf(M, xor_lane<4>(M));
    M = fmaxf(M, xor_lane<8>(M));
    M = max16(M);
    if (h2 < G && jj == 0) C.M[h2] = M;
  }
  __syncthreads();
  for (int i = tid(); i < ns * G; i += MK_WG_THREADS) {
    const int s = i / G, h2 = i % G;
    const float ms = C.f[s][h2];
    C.f[s][h2] = ms == kNegInf ? 0.f : __expf(ms - C.M[h2]);
  }
  __syncthreads();
  {
    const int h2 = tid() >> 5, jj = tid() & 31;
    float L = 0.f;
    if (h2 < G)
      for (int s = jj; s < ns; s += 32) L = fmaf(C.f[s][h2], C.l[s][h2], L);
    L = group_sum(L, 32);
    if (h2 < G && jj == 0) C.L[h2] = L;
  }
  mark(sm, 2);
  const size_t dst_off = (size_t)b * P.QH * D + (size_t)g * G * D;
  const Pub dst_h(o_of(P, 0) + dst_off), dst_l(o_of(P, 1) + dst_off);
  float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
  if (part < NP) {
    for (int s0 = part; s0 < ns; s0 += NP * SB) {
      if (s0 != part) {
#pragma unroll
        for (int k = 0; k < SB; ++k) {
          const int s = s0 + k * NP;
          v[k] = s < ns ? src.ldf4(s * stride + 4 * j) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
#pragma unroll
      for (int k = 0; k < SB; ++k) {
        const int s = s0 + k * NP;
        if (s < ns) {
          const float f = C.f[s][hh];
          O.x = fmaf(f, v[k].x, O.x);
          O.y = fmaf(f, v[k].y, O.y);
          O.z = fmaf(f, v[k].z, O.z);
          O.w = fmaf(f, v[k].w, O.w);
        }
      }
    }
  }
  C.part[tid()] = O;
  __syncthreads();
  if (tid() < GD4) {
    float4 t = C.part[tid()];
    for (int q = 1; q < NP; ++q) {
      const float4 u = C.part[q * GD4 + tid()];
      t.x += u.x;
      t.y += u.y;
      t.z += u.z;
      t.w += u.w;
    }
    // the O projection's matrix-core operand, as a split pair
    const float inv = 1.f / C.L[hh];
    const float r[4] = {t.x * inv, t.y * inv, t.z * inv, t.w * inv};
    uint16_t h[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split_bf16(r[i], h[i], lo[i]);
    const u32x2_t vh = {(uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
    const u32x2_t vl = {(uint32_t)lo[0] | ((uint32_t)lo[1] << 16), (uint32_t)lo[2] | ((uint32_t)lo[3] << 16)};
    if (lds_h) {  // the consumer's own operand (group-relative)
      *(u32x2_t*)(lds_h + 4 * j) = vh;
      *(u32x2_t*)(lds_l + 4 * j) = vl;
    }
    if (to_global) {
      dst_h.st16x4(4 * j, vh);
      dst_l.st16x4(4 * j, vl);
    }
  }
}

// ---------------------------------------------------------------- embed
// Layer 0's input for one column block: h = Emb[token] for every sequence,
// u = bf16(h * gamma_0) and the block's per-token sum of squares.
__device__ __forceinline__ void write_block_input(const mk_params& P, int l_next, int cb, const float* hv,
                                                  const float* gv, int n, Smem& sm);

__device__ __forceinline__ void op_embed(const mk_params& P, const mk_task& t, Smem& sm) {
  const int cb = t.a[0];
  const int H = P.H, CB = P.CB, n = P.B * CB;
  constexpr int NI = MK_MAX_BATCH * 64 / MK_WG_THREADS;  // elements per thread (CB <= 64)
  float hv[NI], gv[NI];
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    const int idx = tid() + k * MK_WG_THREADS;
    hv[k] = gv[k] = 0.f;
    if (idx < n) {
      const int b = idx / CB, c = cb * CB + idx % CB;
      int tok = P.tokens[b];
      if (tok < 0 || tok >= P.V) {
        raise_error(P, MK_DEVERR_FAULT, 1000 + b, (uint32_t)tok);
        tok = 0;
      }
      hv[k] = bf2f(P.emb[(size_t)tok * H + c]);
      gv[k] = bf2f(P.gamma[c]);
    }
  }
  write_block_input(P, 0, cb, hv, gv, n, sm);
  arrive_nr(P, t.sig_ctr[0]);
}

// Store the residual stream of column block cb (hv[k] = element idx =
// tid() + k * 512 of the block, row idx / CB), the next layer's input
// u = bf16(h * gamma_{l_next}) (gv[k]: the element's gamma) and the block's
// per-token sum of squares.
__device__ __forceinline__ void write_block_input(const mk_params& P, int l_next, int cb, const float* hv,
                                                  const float* gv, int n, Smem& sm) {
  const int H = P.H, CB = P.CB;
  constexpr int NI = MK_MAX_BATCH * 64 / MK_WG_THREADS;
  const Pub h(P.h), Uh(u_of_w(P, l_next, 0)), Ul(u_of_w(P, l_next, 1));
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    const int idx = tid() + k * MK_WG_THREADS;
    if (idx < n) {
      const int b = idx / CB, c = cb * CB + idx % CB;
      h.stf(b * H + c, hv[k]);
      uint16_t hi, lo;
      split_bf16(hv[k] * gv[k], hi, lo);
      Uh.st16(b * H + c, hi);
      Ul.st16(b * H + c, lo);
    }
    // the row's sum of squares across its CB lanes (a row never straddles
    // a wave: CB divides 64), butterfly order; waves past the block's
    // elements skip it (each step is a dependent LDS exchange)
    if (wave_id() * 64 + k * MK_WG_THREADS < n) {
      float sq = idx < n ? hv[k] * hv[k] : 0.f;
      sq = group_sum(sq, CB);
      if (idx < n && idx % CB == 0) Pub(ssq_of(P, l_next)).stf((idx / CB) * P.NB + cb, sq);
    }
  }
}

// -------------------------------------------------------------------- QKV
// QKV panels with RoPE in the epilogue and the K/V append into the paged
// cache (megakernel post, section "Tasks": QKV_PROJ applies RoPE in-register
// in its epilogue; tiny-vllm walkthrough: the new token's K/V are written to
// page block_table[pos / 16], slot pos % 16, before attention reads them).
template <int MT, int NCH>
__device__ __forceinline__ void op_qkv(const mk_params& P, const mk_task& t, Smem& sm) {
  const int l = t.layer, p0 = t.a[0], np = t.a[1];
  // This thread's k-th output, element o of the reduced tiles (panel o / 256,
  // token o / 16 % 16, column o % 16). One row tile: a bijection that gives
  // the outputs of tokens 0-3 ([0, 64) and [256, 320)) to waves 6 and 7, so
  // at batches up to MK_FUSED_B the other waves issue no stores and the next
  // task's loads on them do not retire behind these (the memory counter
  // retires in order).
  auto qkv_out = [&](int k) -> int {
    const int x = tid();
    if constexpr (MT == 1) return x < 192 ? x + 64 : x < 384 ? x + 128 : x < 448 ? x - 384 : x - 192;
    return x + k * MK_WG_THREADS;
  };
  const int kc = P.H / 32;
  const size_t pstride = (size_t)kc * 512;
  const int qd = P.QH * P.D, kvd = P.KVH * P.D, D = P.D, PS = P.PS;
  // Each thread's outputs (2 MT of them, element o = tid + k * 512 of the
  // reduced tiles): the token's length, its page and, for q and k columns,
  // the RoPE factors depend on no activation, so they load before the
  // weights and the wait, and the epilogue after the products only computes
  // and stores.
  constexpr int NO = 2 * MT * 256 / MK_WG_THREADS;
  int seq[NO], page[NO];
  float rc[NO], rs[NO];
#pragma unroll
  for (int k = 0; k < NO; ++k) {
    const int o = qkv_out(k);
    const int pp = o / (MT * 256), mt = (o / 256) % MT, m = (o / 16) % 16;
    const int b = mt * 16 + m;
    seq[k] = (pp < np && b < P.B) ? P.seq_lens[b] : 0;
  }
#pragma unroll
  for (int k = 0; k < NO; ++k) {
    const int o = qkv_out(k);
    const int pp = o / (MT * 256), mt = (o / 256) % MT, m = (o / 16) % 16, nn = o % 16;
    const int b = mt * 16 + m;
    const int n = (p0 + pp) * 16 + nn;
    const bool ok = seq[k] >= 1 && seq[k] <= P.max_seq;
    const int pos = ok ? seq[k] - 1 : 0;
    page[k] = ok ? P.bt[b * P.mpps + pos / PS] : -1;
    const int d = (n < qd ? n : n - qd) % D;
    const bool rot = ok && n < qd + kvd;
    rc[k] = rot ? P.rope[((size_t)pos * (D / 2) + d / 2) * 2 + 0] : 0.f;
    rs[k] = rot ? P.rope[((size_t)pos * (D / 2) + d / 2) * 2 + 1] : 0.f;
  }
  WTile<2, NCH> w;
  wtile_load(w, P.wqkv + l * P.s_wqkv + (size_t)p0 * pstride, pstride, np, 0, kc);
  if (!wait_task(P, t, sm)) return;
  set_rows_batch(P, sm, 0, P.H, 0);
  __syncthreads();
  ATile<MT, NCH> Ah, Al;
  atile_load_bf16(Ah, Pub(u_of(P, l, 0)), sm.row_off[0], 0, kc);
  atile_load_bf16(Al, Pub(u_of(P, l, 1)), sm.row_off[0], 0, kc);
  load_inv_rms(P, l, sm);
  mark(sm, 0);
  Acc<2, MT> acc;
  mfma_tiles(acc, w, Ah, Al);
  reduce_tiles(acc, sm);
  mark(sm, 1);
  const Pub KV(P.kv + l * P.s_kv_l), Q(P.q), QT(P.qt), KVT(P.kvt);
  const bool tg = P.tagged != 0;
  const uint32_t tag = step_tag(P, l);
#pragma unroll
  for (int k = 0; k < NO; ++k) {
    const int o = qkv_out(k);
    const int pp = o / (MT * 256), mt = (o / 256) % MT, m = (o / 16) % 16, nn = o % 16;
    const int b = mt * 16 + m;
    if (pp >= np || b >= P.B) continue;
    if (seq[k] < 1 || seq[k] > P.max_seq) {
      raise_error(P, MK_DEVERR_FAULT, 2000 + b, (uint32_t)seq[k]);
      continue;
    }
    const float inv = sm.inv_rms[b];
    const float y = sm.out[o] * inv, yp = sm.out[o ^ 1] * inv;  // o ^ 1: the pair partner column
    const int pos = seq[k] - 1;
    const int n = (p0 + pp) * 16 + nn;
    const bool odd = n & 1;
    const bool page_ok = page[k] >= 0 && page[k] < P.n_pages;
    if (n < qd + kvd) {
      const int d = (n < qd ? n : n - qd) % D;
      const float c = rc[k], sn = rs[k];
      // pair (x0, x1) -> (x0 c - x1 s, x0 s + x1 c)
      const float x0 = odd ? yp : y, x1 = odd ? y : yp;
      const float r = odd ? (x0 * sn + x1 * c) : (x0 * c - x1 * sn);
      if (n < qd) {
        if (tg)
          QT.st_tagged(b * qd + n, __float_as_uint(r), tag);
        else
          Q.stf(b * qd + n, r);
      } else {
        const int g = (n - qd) / D;
        const uint32_t kb = f2bf(r);
        if (page_ok) KV.st16(((page[k] * 2 + 0) * P.KVH + g) * PS * D + (pos % PS) * D + d, (uint16_t)kb);
        if (tg) KVT.st_tagged(((b * P.KVH + g) * 2 + 0) * D + d, kb, tag);
      }
    } else {
      const int nn2 = n - qd - kvd;
      const int g = nn2 / D, d = nn2 % D;
      const uint32_t vb = f2bf(y);
      if (page_ok) KV.st16(((page[k] * 2 + 1) * P.KVH + g) * PS * D + d * PS + (pos % PS), (uint16_t)vb);
      if (tg) KVT.st_tagged(((b * P.KVH + g) * 2 + 1) * D + d, vb, tag);
    }
    if (!page_ok) raise_error(P, MK_DEVERR_FAULT, 3000 + b, (uint32_t)page[k]);
  }
  // (tagged: attention polls the words; the stores retire on their own, and
  // the next task on this unit does not wait for them: only waves 6 and 7
  // stored at batches up to MK_FUSED_B)
  if (!tg) arrive_nr(P, t.sig_ctr[0]);
}

// ------------------------------------------------------------- residual
// Residual add of one column block, done by whichever contribution to the
// block arrives last (the KVH O-projection partials and the block's tile of
// every routed expert's down projection): h += sum_g a_g + sum_j w_j y_j per
// token, the experts summed in rank order (MOE_COMBINE), then the next
// layer's input u and the block's sums of squares (the fused residual add +
// RMSNorm of the megakernel post, section "Reduce wave quantization").
// The routing weights are in sm.tkw.
__device__ __forceinline__ void residual_block(const mk_params& P, int l, int cb, Smem& sm) {
  const int H = P.H, K = P.K, CB = P.CB, B = P.B, n = B * CB;
  constexpr int NI = MK_MAX_BATCH * 64 / MK_WG_THREADS;
  const Pub h(P.h), ao(P.ao), dn(P.dn);
  const uint16_t* gam = P.gamma + (size_t)(l + 1) * H;
  float hv[NI], gv[NI];
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    const int idx = tid() + k * MK_WG_THREADS;
    hv[k] = gv[k] = 0.f;
    if (idx < n) {
      gv[k] = bf2f(gam[cb * CB + idx % CB]);
      const int b = idx / CB, c = cb * CB + idx % CB;
      // every load in flight before the sums (fixed order: groups, then ranks)
      float av[MK_MAX_KVH], yv[MK_MAX_TOPK];
#pragma unroll
      for (int g = 0; g < MK_MAX_KVH; ++g) av[g] = g < P.KVH ? ao.ldf((g * B + b) * H + c) : 0.f;
#pragma unroll
      for (int j = 0; j < MK_MAX_TOPK; ++j) yv[j] = j < K ? dn.ldf((b * K + j) * H + c) : 0.f;
      const float h0 = h.ldf(b * H + c);
      float a = 0.f;
#pragma unroll
      for (int g = 0; g < MK_MAX_KVH; ++g)
        if (g < P.KVH) a += av[g];
      float y = 0.f;
#pragma unroll
      for (int j = 0; j < MK_MAX_TOPK; ++j)
        if (j < K) y = fmaf(sm.tkw[b * K + j], yv[j], y);
      hv[k] = (h0 + a) + y;
    }
  }
  write_block_input(P, l + 1, cb, hv, gv, n, sm);
}

// After a contribution to column block cb: the last of the block's
// KVH + n_active contributions does the residual and signals the next layer.
// The arrival, the active-expert count and the routing weights travel in one
// round trip.
__device__ __forceinline__ void block_arrive(const mk_params& P, const mk_task& t, int ctr_base, int cb, Smem& sm) {
  sync_published();
  const int i = tid();
  if (i == 0) sm.old = (int)__hip_atomic_fetch_add(&P.ctr[ctr_base + cb], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (i == 64) sm.t_old[0] = Pub(route_of(P, t.layer)).ldi(0);
  const float w = i < P.B * P.K ? Pub(tkw_of(P, t.layer)).ldf(i) : 0.f;  // B * K <= 512
  __syncthreads();
  const int old = sm.old, n_active = sm.t_old[0];
  if (old == P.KVH + n_active - 1) {
    if (i < P.B * P.K) sm.tkw[i] = w;
    __syncthreads();
    residual_block(P, t.layer, cb, sm);
    arrive_nr(P, t.sig_ctr[0]);
  }
  __syncthreads();
}

// ------------------------------------------------------------------ O proj
// O projection split-K by kv group: group g's heads contribute their slice
// of the K dimension as soon as that group's attention lands (megakernel
// post, section "Drop false dependencies"); one task per (group, column block),
// or (NPO = 8, a[3] = 2) per (group, two adjacent column blocks), whose 256 KB
// of weights all stream before the wait.
// MERGE (at most MK_FUSED_B tokens): the task waits for the group's attention
// splits (a[4] of them per sequence) and merges them itself into its operand
// in LDS (ATTN_COMBINE inside the projection), so no compute unit combines
// first; the first block's task also stores the merged attention output.
template <int D, int MT, int NCH, int NPO, bool MERGE>
__device__ __forceinline__ void op_oproj(const mk_params& P, const mk_task& t, Smem& sm) {
  const int l = t.layer, g = t.a[0], cb = t.a[1], nblk = NPO == 8 ? t.a[3] : 1;
  const int DP = P.CB / 16, p0 = cb * DP, np = DP * nblk;
  const int kc = P.QH * P.D / 32;
  const int c0 = g * P.G * P.D / 32, c1 = c0 + P.G * P.D / 32;
  const size_t pstride = (size_t)kc * 512;
  WTile<NPO, NCH> w;
  wtile_load(w, P.wo + l * P.s_wo + (size_t)p0 * pstride, pstride, np, c0, c1);
  if (!wait_task(P, t, sm)) return;
  mark(sm, 0);
  ATile<MT, NCH> Ah, Al;
  if constexpr (MERGE) {
    const int GD = P.G * D;  // <= 1024
    uint16_t* oh = sm.act;
    uint16_t* ol = sm.act + MK_FUSED_B * 1024;
    for (int b = 0; b < P.B; ++b) {
      attn_combine<D, 8, 1>(P, b, g, t.a[4], sm, oh + b * GD, ol + b * GD, cb == 0);
      __syncthreads();
    }
    const int wv = wave_id(), ln = lane_id(), row = ln & 15;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int cr = wv + MK_WAVES * i;  // chunk relative to the group's first
      const bool ok = cr < c1 - c0 && row < P.B;
      Ah.a[0][i] = ok ? *(const u32x4_t*)(oh + row * GD + 32 * cr + 8 * (ln >> 4)) : u32x4_t{0u, 0u, 0u, 0u};
      Al.a[0][i] = ok ? *(const u32x4_t*)(ol + row * GD + 32 * cr + 8 * (ln >> 4)) : u32x4_t{0u, 0u, 0u, 0u};
    }
  } else {
    set_rows_batch(P, sm, 0, P.QH * P.D, 0);
    __syncthreads();
    atile_load_bf16(Ah, Pub(o_of(P, 0)), sm.row_off[0], c0, c1);
    atile_load_bf16(Al, Pub(o_of(P, 1)), sm.row_off[0], c0, c1);
  }
  Acc<NPO, MT> acc;
  mfma_tiles(acc, w, Ah, Al);
  reduce_tiles(acc, sm);
  mark(sm, 1);
  const Pub AO(P.ao);
  for (int o = tid(); o < NPO * MT * 256; o += MK_WG_THREADS) {
    const int pp = o / (MT * 256), mt = (o / 256) % MT, m = (o / 16) % 16, nn = o % 16;
    const int b = mt * 16 + m;
    if (pp < np && b < P.B) AO.stf((g * P.B + b) * P.H + (p0 + pp) * 16 + nn, sm.out[o]);
  }
  if (t.b[0] == 1)
    arrive_nr(P, t.a[2]);  // fused MoE: a residual task sums the block
  else
    block_arrive(P, t, t.a[2], cb, sm);
}

// ------------------------------------------------------------------ router
// Router logits over a K range of a panel range (partial sums); the task that
// completes the router does ROUTER_TOPK + ROUTE_FINALIZE (megakernel post,
// section "Tasks"): sum the partials in fixed order, top-k (ties to the lower
// expert index), softmax over the kept logits, the expert work queue.
__device__ __forceinline__ bool route_build(const mk_params& P, int l, Smem& sm, bool publish);
__device__ __forceinline__ bool route_rank(const mk_params& P, int l, Smem& sm, bool publish, int& n_active);
__device__ __forceinline__ void route_finish(const mk_params& P, int l, Smem& sm, bool publish, int n_active);
__device__ __forceinline__ void route_trivial(const mk_params& P, int l, Smem& sm, bool norm);
__device__ __forceinline__ void topk_finalize(const mk_params& P, int l, Smem& sm);

template <int MT, int NCH>
__device__ __forceinline__ void op_router(const mk_params& P, const mk_task& t, Smem& sm) {
  const int l = t.layer, p0 = t.a[0], np = t.a[1], c0 = t.a[2], c1 = t.a[3], ks = t.a[4];
  const int kc = P.H / 32;
  const size_t pstride = (size_t)kc * 512;
  WTile<2, NCH> w;
  wtile_load(w, P.wr + l * P.s_wr + (size_t)p0 * pstride, pstride, np, c0, c1);
  if (!wait_task(P, t, sm)) return;
  set_rows_batch(P, sm, 0, P.H, 0);
  __syncthreads();
  ATile<MT, NCH> Ah, Al;
  atile_load_bf16(Ah, Pub(u_of(P, l, 0)), sm.row_off[0], c0, c1);
  atile_load_bf16(Al, Pub(u_of(P, l, 1)), sm.row_off[0], c0, c1);
  load_inv_rms(P, l, sm);
  mark(sm, 0);
  Acc<2, MT> acc;
  mfma_tiles(acc, w, Ah, Al);
  reduce_tiles(acc, sm);
  mark(sm, 1);
  const Pub RP(rp_of(P, l)), RPT(P.rpt);
  const bool tg = P.tagged != 0;
  const uint32_t tag = step_tag(P, l);
  for (int o = tid(); o < 2 * MT * 256; o += MK_WG_THREADS) {
    const int pp = o / (MT * 256), mt = (o / 256) % MT, m = (o / 16) % 16, nn = o % 16;
    const int b = mt * 16 + m, e = (p0 + pp) * 16 + nn;
    if (pp < np && b < P.B && e < P.E) {
      const float v = sm.out[o] * sm.inv_rms[b];
      RP.stf((ks * P.B + b) * P.E + e, v);
      // (tagged: the fused MoE claimers poll these; the arrival below is for
      // the task that publishes the route)
      if (tg) RPT.st_tagged((b * P.E + e) * 4 + ks, __float_as_uint(v), tag);
    }
  }
  const int old = arrive(P, t.a[5], sm);
  if (old == P.n_router_tasks - 1) {
    mark(sm, 2);
    topk_finalize(P, l, sm);
    mark(sm, 3);
    arrive_nr(P, t.sig_ctr[0]);
  }
}

// Top-k by ranking: expert e's rank for token b is the number of experts
// ahead of it (a larger logit, or an equal logit and a lower index); the
// experts ranked below k are kept, in rank order. Every comparison is
// independent, so this takes a few hundred cycles per token instead of k
// dependent rounds of an argmax. Then the route: the active experts in
// ascending order, the tokens routed to each, and the work-item counts, built
// in LDS (sm.rt_*, the routing weights in sm.tkw) and, with publish, stored for
// the other compute units. Without publish, layer l's sums of squares load
// alongside the router logits (then sm.inv_rms).
// In two parts: route_rank (the logits, each token's top k, the active
// experts in ascending order with their token counts, and their number) and
// route_finish (the routing weights, each active expert's slots, the header
// and, without publish, the layer input's 1/rms); a fused claimer issues its
// first item's weights between them.
__device__ __forceinline__ bool route_build(const mk_params& P, int l, Smem& sm, bool publish) {
  int n_active = 0;
  const bool ok = route_rank(P, l, sm, publish, n_active);
  route_finish(P, l, sm, publish, n_active);
  return ok;
}

__device__ __forceinline__ bool route_rank(const mk_params& P, int l, Smem& sm, bool publish, int& n_active) {
  const int E = P.E, K = P.K, B = P.B;
  const Pub R(rp_of(P, l)), RT(route_of(P, l)), RPT(P.rpt);
  SmemTopk& T = sm.u.tk;
  // a fused claimer with tagged hand-offs polls the partials' tagged words
  // (sm.flag is 1 from its wait and drops to 0 on a failed poll)
  const bool poll = !publish && P.tagged != 0;
  const uint32_t tag = step_tag(P, l);
  float sq[2];  // B * NB <= 1024
  if (!publish) {
    const Pub S(ssq_of(P, l));
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = tid() + k * MK_WG_THREADS;
      sq[k] = i < B * P.NB ? S.ldf(i) : 0.f;
    }
  }
  for (int i = tid(); i < B * E; i += MK_WG_THREADS) {
    float p[MK_MAX_RKS];
    if (poll) {
      const int ks = P.router_ks;
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      uint32_t spins = 0;
      u32x4_t a = RPT.ld_tagged2(4 * i), c = RPT.ld_tagged2(4 * i + 2);
      while (!((a[1] == tag || ks < 1) && (a[3] == tag || ks < 2) && (c[1] == tag || ks < 3) &&
               (c[3] == tag || ks < 4))) {
        __builtin_amdgcn_s_sleep(1);
        if ((++spins & 63u) == 0) {
          if (ld_relaxed(&P.err[0]) != 0) {
            sm.flag = 0;
            break;
          }
          if ((int64_t)(__builtin_amdgcn_s_memrealtime() - t0) > P.timeout_ticks) {
            raise_error(P, MK_DEVERR_TIMEOUT, 0xffff0000u | (uint32_t)(4 * i), a[1]);
            sm.flag = 0;
            break;
          }
        }
        a = RPT.ld_tagged2(4 * i);
        c = RPT.ld_tagged2(4 * i + 2);
      }
      p[0] = __uint_as_float(a[0]);
      p[1] = __uint_as_float(a[2]);
      p[2] = __uint_as_float(c[0]);
      p[3] = __uint_as_float(c[2]);
    } else {
#pragma unroll
      for (int k = 0; k < MK_MAX_RKS; ++k) p[k] = k < P.router_ks ? R.ldf(k * B * E + i) : 0.f;
    }
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < MK_MAX_RKS; ++k)
      if (k < P.router_ks) v += p[k];
    const int b = i / E, e = i % E;
    T.logit[b][e] = v;
    // a 64-bit key ordered like (logit, -index): the float's bits made
    // monotone as an unsigned integer (-0 taken as +0, so equal logits tie
    // and go by index), then the complemented index
    const uint32_t u = v == 0.f ? 0u : __float_as_uint(v);
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    T.key[b][e] = ((uint64_t)ord << 32) | (uint32_t)(0xffffu - e);
  }
  // keys past the last expert of each row: zero, below every real key
  for (int i = tid(); i < B * 128; i += MK_WG_THREADS)
    if (i % 128 >= E) T.key[i / 128][i % 128] = 0ull;
  if ((int)tid() < E) T.tokmask[tid()] = 0u;
  if (!publish) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = tid() + k * MK_WG_THREADS;
      if (i < B * P.NB) sm.ssq[i] = sq[k];
    }
  }
  lds_sync();
  // rank of (b, e): the keys above its own
  auto keep = [&](int b, int e, int rank) {
    if (rank < K) {
      T.sel_idx[b][rank] = e;
      T.sel_val[b][rank] = T.logit[b][e];
      // route: each expert's set of tokens as a bit mask (a token keeps an
      // expert at most once)
      atomicOr(&T.tokmask[e], 1u << b);
    }
  };
  if (B >= MK_WAVES) {
    // a wave per token: each lane ranks experts lane and lane + 64 against
    // every key of the row, read as broadcasts (one address for the wave)
    const int e0 = lane_id(), e1 = lane_id() + 64;
    for (int b = wave_id(); b < B; b += MK_WAVES) {
      const uint64_t me0 = T.key[b][e0], me1 = T.key[b][e1];
      int r0 = 0, r1 = 0;
#pragma unroll 8
      for (int j = 0; j < 128; j += 2) {
        const uint64_t k0 = T.key[b][j], k1 = T.key[b][j + 1];
        r0 += (k0 > me0) + (k1 > me0);
        r1 += (k0 > me1) + (k1 > me1);
      }
      if (e0 < E) keep(b, e0, r0);
      if (e1 < E) keep(b, e1, r1);
    }
  } else {
    // four threads per pair, thread q over the experts j with j % 4 == q (the
    // four lanes of a pair read adjacent keys: no bank conflicts), summed
    // across the four adjacent lanes
    for (int i = tid(); i < B * E * 4; i += MK_WG_THREADS) {
      const int q = i & 3, pe = i >> 2, b = pe / E, e = pe % E;
      const uint64_t me = T.key[b][e];
      int rank = 0;
#pragma unroll 4
      for (int j = 0; j < 128; j += 8) {
        const uint64_t k0 = T.key[b][j + q], k1 = T.key[b][j + 4 + q];
        rank += (k0 > me) + (k1 > me);
      }
      rank += xor_lane<1>(rank);
      rank += xor_lane<2>(rank);
      if (q == 0) keep(b, e, rank);
    }
  }
  lds_sync();
  // the experts' positions among the active ones from two wave ballots, and
  // each slot's rank within its expert (tokens in ascending order)
  if (tid() < 128) {
    const int e = tid();
    const bool act = e < E && T.tokmask[e] != 0u;
    const uint64_t bal = __ballot(act);
    if (lane_id() == 0) T.ballot[e >> 6] = bal;
  }
  lds_sync();
  const uint64_t b0 = T.ballot[0], b1 = E > 64 ? T.ballot[1] : 0ull;
  n_active = __popcll(b0) + __popcll(b1);
  if ((int)tid() < E) {
    const int e = tid();
    const uint32_t mask = T.tokmask[e];
    const int a = e < 64 ? __popcll(b0 & ((1ull << e) - 1ull)) : __popcll(b0) + __popcll(b1 & ((1ull << (e - 64)) - 1ull));
    T.apos[e] = a;
    if (mask) {
      sm.rt_e[a] = e;
      sm.rt_cnt[a] = __popc(mask);
      if (publish) {
        RT.sti(4 + a, e);
        RT.sti(4 + E + a, __popc(mask));
      }
    }
  }
  lds_sync();
  return !poll || sm.flag != 0;
}

__device__ __forceinline__ void route_finish(const mk_params& P, int l, Smem& sm, bool publish, int n_active) {
  const int E = P.E, K = P.K, B = P.B;
  const Pub TI(tki_of(P, l)), TW(tkw_of(P, l)), RT(route_of(P, l));
  SmemTopk& T = sm.u.tk;
  if (!publish) inv_rms_lds(P, sm);
  for (int i = tid(); i < B * K; i += MK_WG_THREADS) {
    // softmax over the kept logits (max-subtracted; rank 0 is the max),
    // summed in rank order
    const int b = i / K, j = i % K;
    const float top = T.sel_val[b][0];
    float sum = 0.f;
    for (int jj = 0; jj < K; ++jj) sum += __expf(T.sel_val[b][jj] - top);
    const float w = __expf(T.sel_val[b][j] - top) / sum;
    sm.tkw[i] = w;
    if (publish) {
      TI.sti(i, T.sel_idx[b][j]);
      TW.stf(i, w);
      if (P.tk_trace) P.tk_trace[((size_t)l * B + b) * K + j] = T.sel_idx[b][j];
    }
  }
  for (int i = tid(); i < B * K; i += MK_WG_THREADS) {
    const int b = i / K, e = T.sel_idx[b][i % K];
    const int r = __popc(T.tokmask[e] & ((1u << b) - 1u));
    sm.rt_slot[T.apos[e] * B + r] = i;
    if (publish) RT.sti(4 + 2 * E + T.apos[e] * B + r, i);
  }
  if (tid() == 0) {
    sm.rt_hdr[0] = n_active;
    sm.rt_hdr[1] = n_active * P.up_items_per_expert;
    sm.rt_hdr[2] = n_active * P.down_items_per_expert;
    if (publish) {
      RT.sti(0, n_active);
      RT.sti(1, n_active * P.up_items_per_expert);
      RT.sti(2, n_active * P.down_items_per_expert);
    }
  }
  lds_sync();
}

__device__ __forceinline__ void topk_finalize(const mk_params& P, int l, Smem& sm) { route_build(P, l, sm, true); }

// A claimer's start in one round trip: the first claim of n items (thread 0;
// the result in sm.claim; none with claim_ctr < 0), the route entries of the layer's active experts
// and, with l >= 0, the sums of squares of layer l's input (then sm.inv_rms).
__device__ __forceinline__ void claimer_start(const mk_params& P, int32_t claim_ctr, int n, int l, Smem& sm,
                                              int32_t claim2_ctr = -1, int n2 = 1) {
  const Pub R(route_of(P, l));
  const int E = P.E, B = P.B;
  const int i = tid();
  int c = 0;
  if (i == 0 && claim_ctr >= 0)
    c = (int)__hip_atomic_fetch_add(&P.ctr[claim_ctr], (uint32_t)n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (i == 64 && claim2_ctr >= 0)
    sm.claim2 = (int)__hip_atomic_fetch_add(&P.ctr[claim2_ctr], (uint32_t)n2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (i < 4) sm.rt_hdr[i] = R.ldi(i);
  if (i < E) {
    sm.rt_e[i] = R.ldi(4 + i);
    sm.rt_cnt[i] = R.ldi(4 + E + i);
  }
  for (int k = i; k < E * B; k += MK_WG_THREADS) sm.rt_slot[k] = R.ldi(4 + 2 * E + k);
  if (i < B * P.K) sm.tkw[i] = Pub(tkw_of(P, l)).ldf(i);
  if (l >= 0) {
    const Pub S(ssq_of(P, l));
    for (int k = i; k < B * P.NB; k += MK_WG_THREADS) sm.ssq[k] = S.ldf(k);
  }
  if (i == 0) sm.claim = c;
  __syncthreads();
  if (l >= 0) inv_rms_lds(P, sm);
  __syncthreads();
}

// ------------------------------------------------------------------ MoE
// Expert up/gate over one K half of one gate/up panel pair for all tokens
// routed to the expert, claimed from the queue ROUTER_TOPK built (megakernel
// post, section "Tasks": MOE_UPGATE_ACT_DRAIN; the scheduler section of the
// Chinese version: claimers take the next entry atomically until the queue is
// empty). The two K halves' gate and up sums are added, and the
// SiLU-and-multiply applied, by the down projection that consumes them.
// Claims take several items at a time (their weights stream together); the
// batch size spreads the queue over the claimers expected to be free.
template <int MT, int NCH>
__device__ __forceinline__ void down_item(const mk_params& P, const mk_task& t, int a, int cb, const WTile<4, NCH>& w,
                                          Smem& sm, bool stage = true);
template <int MT, int NPR>
__device__ __forceinline__ void down_item(const mk_params& P, const mk_task& t, int a, int cb,
                                          const WTile8<4, NPR>& w, Smem& sm, bool stage = true);

// The claiming MoE above 16 tokens: each up/gate item's matrix-core rows are
// the tokens routed to its expert (a second 16-row tile when an expert has
// more), loaded together with the item's weights, so an item's operand takes
// one row tile of registers instead of the whole batch's two and two items'
// weights stream at once. Down items as in the claiming variant.
// One O-projection item of a claiming MoE claimer: group g's K slice of column
// block cb for every token (the product op_oproj runs above MK_FUSED_B
// tokens), once the group's combined attention output is complete (counter
// b[0] + g, target b[1]); its contribution counts on the block's counter,
// and the last contribution to the block does its residual.
template <int MT>
__device__ __forceinline__ void oproj_item(const mk_params& P, const mk_task& t, int g, int cb, Smem& sm) {
  constexpr int NCH = 32 / MK_WAVES, NPO = 4;
  const int l = t.layer;
  const int DP = P.CB / 16, p0 = cb * DP;
  const int kc = P.QH * P.D / 32;
  const int c0 = g * P.G * P.D / 32, c1 = c0 + P.G * P.D / 32;
  const size_t pstride = (size_t)kc * 512;
  WTile<NPO, NCH> w;
  wtile_load(w, P.wo + l * P.s_wo + (size_t)p0 * pstride, pstride, DP, c0, c1);
  if (!wait_one(P, t.b[0] + g, t.b[1], sm)) return;
  set_rows_batch(P, sm, 0, P.QH * P.D, 0);
  __syncthreads();
  ATile<MT, NCH> Ah, Al;
  atile_load_bf16(Ah, Pub(o_of(P, 0)), sm.row_off[0], c0, c1);
  atile_load_bf16(Al, Pub(o_of(P, 1)), sm.row_off[0], c0, c1);
  Acc<NPO, MT> acc;
  mfma_tiles(acc, w, Ah, Al);
  reduce_tiles(acc, sm);
  const Pub AO(P.ao);
  for (int o = tid(); o < NPO * MT * 256; o += MK_WG_THREADS) {
    const int pp = o / (MT * 256), mt = (o / 256) % MT, m = (o / 16) % 16, nn = o % 16;
    const int b = mt * 16 + m;
    if (pp < DP && b < P.B) AO.stf((g * P.B + b) * P.H + (p0 + pp) * 16 + nn, sm.out[o]);
  }
  block_arrive(P, t, t.a[4], cb, sm);
}

template <int NCH, int NBMAX, int NCHD, bool FP8 = false, int MT = 2>
__device__ __forceinline__ void op_moe_gather(const mk_params& P, const mk_task& t, Smem& sm) {
  if (!wait_task(P, t, sm)) return;
  const int l = t.layer, claim_ctr = t.a[0], done_base = t.a[1], dclaim_ctr = t.a[3];
  const int F = P.F, upe = P.up_items_per_expert, B = P.B, K = P.K, H = P.H;
  const int kc = H / 32, kh_chunks = kc / 2;
  const size_t pstride = (size_t)kc * 512;
  const Pub GU(P.gu), U0(u_of(P, l, 0)), U1(u_of(P, l, 1));
  // Items are claimed CHU (CHD) at a time; the next chunk's claim is issued when a
  // chunk starts and read when it runs out, so claims (one address shared
  // by every unit) never sit on the path.
  constexpr int CHU = 4, CHD = 4;  // up/gate and down items per claim
  claimer_start(P, claim_ctr, CHU, l, sm, dclaim_ctr, CHD);
  const int n_items = __builtin_amdgcn_readfirstlane(sm.rt_hdr[1]);
  const int n_down = __builtin_amdgcn_readfirstlane(sm.rt_hdr[2]);
  int dbase = sm.claim2;
  if ((int)tid() < 128) sm.done_cnt[tid()] = 0;
  mark(sm, 0);
  // the stream of one queue: the item after the current one (uniform)
  // (current claim: base and size ch; pending claim: pend and size pch)
  struct Stream {
    int base, j, pend, ch, pch, full;
  };
  // (the pending claim is issued unconditionally by thread 0 and read only
  // there, so its result stays in one register: a copy of it, at a join of
  // paths that did and did not claim, would wait for the atomic at once and,
  // the memory counter retiring in order, for every weight load before it.
  // Claims past the queue's end are harmless: their items do not exist.)
  // Near the queue's end the claims shrink to single items, once fewer than
  // two rounds of full claims over every workgroup remain beyond the current
  // one, so the last claimers do not each hold a whole chunk while the others
  // are done.
  auto claim_size = [&](const Stream& q, int n) -> int {
    return n - q.base > 2 * q.full * (int)gridDim.x ? q.full : 1;
  };
  auto stream_start = [&](Stream& q, int base, int32_t ctr, int n, int ch) {
    q.base = base;
    q.j = 0;
    q.ch = q.full = ch;
    q.pch = claim_size(q, n);
    if (tid() == 0)
      q.pend = (int)__hip_atomic_fetch_add(&P.ctr[ctr], (uint32_t)q.pch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  auto stream_next = [&](Stream& q, int32_t ctr, int n) -> int {
    if (++q.j < q.ch) return q.base + q.j;
    if (tid() == 0) sm.claim = q.pend;
    lds_sync();
    q.base = sm.claim;
    lds_sync();
    q.j = 0;
    q.ch = q.pch;
    q.pch = claim_size(q, n);
    if (tid() == 0)
      q.pend = (int)__hip_atomic_fetch_add(&P.ctr[ctr], (uint32_t)q.pch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return q.base;
  };
  // this lane's row of row tile rt of active expert a: the element offset
  // of its token's layer input (-1: past the expert's routed tokens)
  auto row_of = [&](int a, int rt) -> int {
    const int r = rt * 16 + (int)(lane_id() & 15);
    return (a >= 0 && r < sm.rt_cnt[a]) ? (sm.rt_slot[a * B + r] / K) * H : -1;
  };
  // An expert's up/gate items run K half by K half (item r of expert a:
  // K half r / half, gate/up panel pair r % half), so the CHU items of a
  // claimed chunk (claims are CHU-aligned, and half = F / 16 is a multiple of
  // 8 for the supported widths, so a chunk never straddles a K half or an
  // expert) share the routed rows of one K half, loaded once per chunk.
  static_assert(CHU == 4, "one weight slot per item of a chunk");
  const int half = upe / 2;
  // (FP8 feed-forward weights: gate/up codes in chunk pairs, kh_pairs per K
  // half, the routed rows' chunks in the same pair order; the gu partial sums
  // stay unscaled, the down item's staging applies the unit's scales)
  const int kh_pairs = H / 128, pstride8 = (H / 64) * 1024;
  using WG = std::conditional_t<FP8, WTile8<2, NCH / 2>, WTile<2, NCH>>;
  // one item's weights (a zero tile past the queue)
  auto wload = [&](WG& w, int id) {
    const bool valid = id < n_items;
    const int a = valid ? id / upe : 0, r = id % upe;
    const int tt = r % half, kh = r / half;
    const int e = __builtin_amdgcn_readfirstlane(sm.rt_e[a]);
    if constexpr (FP8)
      wtile8_load(w, P.wgu8 + l * P.s_gu8_l + (size_t)e * P.s_gu8_e + (size_t)(2 * tt) * pstride8, pstride8,
                  valid ? 2 : 0, kh * kh_pairs, (kh + 1) * kh_pairs);
    else
      wtile_load(w, P.wgu + l * P.s_wgu_l + (size_t)e * P.s_wgu_e + (size_t)(2 * tt) * pstride, pstride,
                 valid ? 2 : 0, kh * kh_chunks, (kh + 1) * kh_chunks);
  };
  // row tile rt's rows of one K half
  auto row_tile = [&](ATile<1, NCH>& Xh, ATile<1, NCH>& Xl, int o, int kh) {
    if constexpr (FP8) {
      atile_load_row_pairs(Xh, U0, o, kh * kh_pairs, (kh + 1) * kh_pairs);
      atile_load_row_pairs(Xl, U1, o, kh * kh_pairs, (kh + 1) * kh_pairs);
    } else {
      atile_load_row(Xh, U0, o, kh * kh_chunks, (kh + 1) * kh_chunks);
      atile_load_row(Xl, U1, o, kh * kh_chunks, (kh + 1) * kh_chunks);
    }
  };
  // a chunk's routed rows (no rows past the queue)
  auto rows = [&](ATile<1, NCH>& Xh, ATile<1, NCH>& Xl, int id) {
    const bool valid = id < n_items;
    const int a = valid ? id / upe : 0, kh = (id % upe) / half;
    const int o = row_of(valid ? a : -1, 0);
    row_tile(Xh, Xl, o, kh);
  };
  // one item's products and gu stores with its chunk's rows; the arrival is
  // counted in LDS
  auto compute = [&](const WG& w, ATile<1, NCH>& Ah, ATile<1, NCH>& Al, int id) {
    if (id >= n_items) return;
    const int a = id / upe, r = id % upe;
    const int tt = r % half, kh = r / half;
    const int cnt = sm.rt_cnt[a];
    // (at least one row tile: an active expert has a routed token, and the
    // compiler then knows the item's loads are consumed before its registers
    // are loaded again)
    int rt = 0;
    do {
      if (rt > 0)  // an expert with more than 16 routed tokens: the next rows
        row_tile(Ah, Al, row_of(a, rt), kh);
      Acc<2, 1> acc;
      if constexpr (FP8)
        mfma_tiles8(acc, w, Ah, Al, false);
      else
        mfma_tiles(acc, w, Ah, Al);
      reduce_tiles(acc, sm);
      // gu[slot][kh][gate|up][F] of the tile's routed rows
      // (at most 2 x 16 x 16 = 512 values: one predicated store per thread,
      // a count the compiler's memory-counter waits can track; a loop with a
      // run-time trip count made it wait for every store before the next
      // item's loads could be used)
      const int nr = min(16, cnt - rt * 16);
      {
        const int o = tid();
        if (o < 2 * nr * 16) {
          const int which = o / (nr * 16), rr = (o / 16) % nr, nn = o % 16;
          const int slot = sm.rt_slot[a * B + rt * 16 + rr], b = slot / K;
          GU.stf(((slot * 2 + kh) * 2 + which) * F + tt * 16 + nn,
                 sm.out[which * 256 + rr * 16 + nn] * sm.inv_rms[b]);
        }
      }
    } while (++rt * 16 < cnt);
    // (a later item of the chunk needs the first row tile again)
    if (rt > 1 && id % CHU != CHU - 1) row_tile(Ah, Al, row_of(a, 0), kh);
    if (tid() == 0) sm.done_cnt[a] += 1;
  };
  // the next claimed chunk's first item (the claim after it is issued now,
  // read when that chunk starts)
  auto next_chunk = [&](int& pend) -> int {
    if (tid() == 0) sm.claim = pend;
    lds_sync();
    const int base = sm.claim;
    lds_sync();
    if (tid() == 0)
      pend = (int)__hip_atomic_fetch_add(&P.ctr[claim_ctr], (uint32_t)CHU, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return base;
  };
  {
    // four items in flight, one weight slot per item of a chunk: while a
    // chunk's items compute, the next chunk's weights take their slots one by
    // one, and its rows go to the other row set (two chunks per loop pass, so
    // every set index is fixed). The arrivals wait for the end of the phase
    // (one drain), since down items start only after this claimer's up/gate
    // items.
    WG w0, w1, w2, w3;
    ATile<1, NCH> X0h, X0l, X1h, X1l;
    int pend = 0;
    if (tid() == 0)
      pend = (int)__hip_atomic_fetch_add(&P.ctr[claim_ctr], (uint32_t)CHU, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int c0 = sm.claim;
    wload(w0, c0);
    wload(w1, c0 + 1);
    wload(w2, c0 + 2);
    wload(w3, c0 + 3);
    rows(X0h, X0l, c0);
    while (c0 < n_items) {
      const int c1 = next_chunk(pend);
      compute(w0, X0h, X0l, c0);
      wload(w0, c1);
      rows(X1h, X1l, c1);
      compute(w1, X0h, X0l, c0 + 1);
      wload(w1, c1 + 1);
      compute(w2, X0h, X0l, c0 + 2);
      wload(w2, c1 + 2);
      compute(w3, X0h, X0l, c0 + 3);
      wload(w3, c1 + 3);
      if (c1 >= n_items) break;
      c0 = next_chunk(pend);
      compute(w0, X1h, X1l, c1);
      wload(w0, c0);
      rows(X0h, X0l, c0);
      compute(w1, X1h, X1l, c1 + 1);
      wload(w1, c0 + 1);
      compute(w2, X1h, X1l, c1 + 2);
      wload(w2, c0 + 2);
      compute(w3, X1h, X1l, c1 + 3);
      wload(w3, c0 + 3);
    }
  }
  mark(sm, 1);
  sync_published();
  if ((int)tid() < 128 && sm.done_cnt[tid()] > 0)
    __hip_atomic_fetch_add(&P.ctr[done_base + tid()], (uint32_t)sm.done_cnt[tid()], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  // The layer's O projection as a queue of (group, column block) items
  // (a[5] its claim counter; -1: the projection runs as tasks), drained
  // between the up/gate and down phases: by then every group's attention has
  // long completed, and the projection's work joins the balanced claimed
  // work instead of following the slowest claimer on fixed units.
  if (t.a[5] >= 0) {
    const int n_op = P.KVH * P.NB;
    for (int id = claim_n(P, t.a[5], 1, sm); id < n_op; id = claim_n(P, t.a[5], 1, sm)) {
      oproj_item<MT>(P, t, id / P.NB, id % P.NB, sm);
      if (error_seen(error_peek(P), sm)) return;
    }
  }
  mark(sm, 2);
  // down items (two row tiles of routed rows), the next item's weights
  // streaming while the current computes; consecutive items of one expert
  // reuse its staged operand
  const int DP = P.CB / 16, kcd = P.F / 32, dpe = P.down_items_per_expert;
  const size_t pstride_d = (size_t)kcd * 512;
  const int pstride8_d = (P.F / 64) * 1024;
  using WD = std::conditional_t<FP8, WTile8<4, (NCHD + 1) / 2>, WTile<4, NCHD>>;
  auto dload = [&](WD& w, int id) {
    const bool valid = id < n_down;
    const int a = valid ? id / dpe : 0, cb = id % dpe;
    const int e = __builtin_amdgcn_readfirstlane(sm.rt_e[a]);
    if constexpr (FP8)
      wtile8_load(w, P.wd8p + l * P.s_d8_l + (size_t)e * P.s_d8_e + (size_t)(cb * DP) * pstride8_d, pstride8_d,
                  valid ? DP : 0, 0, kcd / 2);
    else
      wtile_load(w, P.wd + l * P.s_wd_l + (size_t)e * P.s_wd_e + (size_t)(cb * DP) * pstride_d, pstride_d,
                 valid ? DP : 0, 0, kcd);
  };
  {
    WD d0, d1;
    Stream q;
    stream_start(q, dbase, dclaim_ctr, n_down, CHD);
    int i0 = q.base;
    dload(d0, i0);
    int i1 = i0 < n_down ? stream_next(q, dclaim_ctr, n_down) : n_down;
    int staged = -1;
    // (the error flag is loaded before the next item's weights and tested
    // after the current item: loaded after them, its test would wait for the
    // whole prefetch, the memory counter retiring in order)
    while (i0 < n_down) {
      uint32_t err = error_peek(P);
      dload(d1, i1);
      down_item<2>(P, t, i0 / dpe, i0 % dpe, d0, sm, i0 / dpe != staged);
      staged = i0 / dpe;
      if (error_seen(err, sm)) return;
      i0 = i1 < n_down ? stream_next(q, dclaim_ctr, n_down) : n_down;
      if (i1 >= n_down) break;
      err = error_peek(P);
      dload(d0, i0);
      down_item<2>(P, t, i1 / dpe, i1 % dpe, d1, sm, i1 / dpe != staged);
      staged = i1 / dpe;
      if (error_seen(err, sm)) return;
      i1 = i0 < n_down ? stream_next(q, dclaim_ctr, n_down) : n_down;
    }
  }
  mark(sm, 3);
}

// The down projection's operand for routed rows [r0, r0 + nr) of active
// expert a: SiLU(gate) * up from the two K halves' partial sums, as the split
// pair in LDS (hi of row r - r0 at act[(r - r0) F + f], lo 16 F further on).
// Only the routed rows are loaded, eight elements per thread in flight per
// round; rows past nr are left as they are (the product's output rows past
// the routed ones are not stored).
// sc: FP8 weights' scale rows of the expert ([F][4]: gate, up, down, 0), or
// null for bf16 weights: then gate and up are scaled before the SiLU and the
// product by the down scale.
__device__ __forceinline__ void stage_act(const mk_params& P, int a, int r0, int nr, Smem& sm,
                                          const float* sc = nullptr) {
  const int F = P.F, B = P.B, n = nr * F, lo = 16 * F;
  const Pub GU(P.gu);
  constexpr int R = 8;
  for (int i0 = tid(); i0 < n; i0 += R * MK_WG_THREADS) {
    float g[R][4];
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int i = i0 + k * MK_WG_THREADS, row = i / F, f = i % F;
      const bool live = i < n;
      const int slot = live ? sm.rt_slot[a * B + r0 + row] : 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) g[k][q] = live ? GU.ldf(((slot * 2 + (q & 1)) * 2 + (q >> 1)) * F + f) : 0.f;
    }
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int i = i0 + k * MK_WG_THREADS;
      if (i < n) {
        float gt = g[k][0] + g[k][1], ut = g[k][2] + g[k][3], dsc = 1.f;
        if (sc) {
          const float4 s4 = *(const float4*)(sc + 4 * (i % F));
          gt *= s4.x;
          ut *= s4.y;
          dsc = s4.z;
        }
        split_bf16(gt / (1.0f + __expf(-gt)) * ut * dsc, sm.act[i], sm.act[lo + i]);
      }
    }
  }
  lds_sync();
}

// One or two (nblk) adjacent column blocks (cb0, cb0 + 1) of one expert's down
// projection for at most 16 routed tokens, each block's weights already in
// registers (the second a zero tile when nblk is 1).
// stage: build the expert's SiLU-and-multiply operand in LDS first (after its
// up/gate items completed); otherwise the operand of the previous pair, the
// same expert, is reused. Each block's arrival may complete its residual.
template <int NCH>
__device__ __forceinline__ void down_pair(const mk_params& P, const mk_task& t, int a, int cb0, int nblk,
                                          const WTile<4, NCH>& w0, const WTile<4, NCH>& w1, bool stage, Smem& sm) {
  const int F = P.F, H = P.H, B = P.B;
  const int kc = F / 32;
  const int DP = P.CB / 16;
  const int cnt = sm.rt_cnt[a];
  const Pub DN(P.dn), GU(P.gu);
  if (stage) {
    if (!wait_one(P, t.a[1] + a, P.up_items_per_expert, sm, true)) return;
    stage_act(P, a, 0, min(cnt, 16), sm);
  }
  Acc<8, 1> acc;
#pragma unroll
  for (int pp = 0; pp < 8; ++pp) acc.c[pp][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int wv = wave_id(), ln = lane_id(), n = 16 * F;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = wv + MK_WAVES * i;
    const int off = (ln & 15) * F + 32 * c + 8 * (ln >> 4);
    const u32x4_t ah = c < kc ? *(const u32x4_t*)(sm.act + off) : u32x4_t{0u, 0u, 0u, 0u};
    const u32x4_t al = c < kc ? *(const u32x4_t*)(sm.act + n + off) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int pp = 0; pp < 8; ++pp) {
      const u32x4_t wv4 = pp < 4 ? w0.v[pp][i] : w1.v[pp - 4][i];
      acc.c[pp][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, al),
                                                             __builtin_bit_cast(bf16x8_t, wv4), acc.c[pp][0], 0, 0, 0);
      acc.c[pp][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ah),
                                                             __builtin_bit_cast(bf16x8_t, wv4), acc.c[pp][0], 0, 0, 0);
    }
  }
  reduce_tiles(acc, sm);
  for (int o = tid(); o < 8 * 256; o += MK_WG_THREADS) {
    const int pp = o / 256, m = (o / 16) % 16, nn = o % 16;
    const int cb = cb0 + pp / 4, p4 = pp % 4;
    if (pp / 4 < nblk && p4 < DP && m < cnt) DN.stf(sm.rt_slot[a * B + m] * H + (cb * DP + p4) * 16 + nn, sm.out[o]);
  }
  // the blocks' arrivals in one round trip
  sync_published();
  if ((int)tid() < nblk)
    sm.t_old[tid()] = (int)__hip_atomic_fetch_add(&P.ctr[t.a[4] + cb0 + tid()], 1u, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
  lds_sync();
  const int last = P.KVH + __builtin_amdgcn_readfirstlane(sm.rt_hdr[0]) - 1;
  const int o0 = sm.t_old[0], o1 = sm.t_old[1];
  lds_sync();
  if (o0 == last) {
    residual_block(P, t.layer, cb0, sm);
    arrive_nr(P, t.sig_ctr[0]);
  }
  if (nblk == 2 && o1 == last) {
    residual_block(P, t.layer, cb0 + 1, sm);
    arrive_nr(P, t.sig_ctr[0]);
  }
}

// The MoE claimer with fixed shares (at most 16 tokens): claimer k takes a
// weighted share of the layer's up/gate items and, among the claimers with
// weight, an equal share of its down items, so no claim round trips to a
// shared counter sit on the path. The
// activation operand loads as soon as the layer input is complete, while the
// route is still pending; up/gate weights stream UPD items deep.
//   b[0] this claimer's index k, b[1] the count nf of claimers (indices first)
//   on compute units without attention work in this layer, b[2] all
//   claimers, b[3] the up/gate weight of the others (of 256);
//   wait_ctr[0]: the layer input, wait_ctr[1]: the router tasks (each
//   claimer takes the top-k and builds the route itself, the same on every
//   compute unit); the other arguments as for the claiming variant.
template <int NCH, int NCHD, int UPD>
__device__ __forceinline__ void op_moe_static(const mk_params& P, const mk_task& t, Smem& sm) {
  // claimers [0, nf) weigh 256, the others wa (all 256 in the kernel-per-op
  // variant, where attention ran in an earlier launch)
  const int sk = t.b[0], nf = t.b[1], nt = t.b[2], wa = P.waits_enabled ? t.b[3] : 256;
  auto pre = [&](int j) -> int64_t { return j <= nf ? (int64_t)j * 256 : (int64_t)nf * 256 + (int64_t)(j - nf) * wa; };
  const int l = t.layer, done_base = t.a[1];
  const int F = P.F, upe = P.up_items_per_expert, B = P.B, K = P.K, E = P.E;
  const int kc = P.H / 32, kh_chunks = kc / 2;
  const size_t pstride = (size_t)kc * 512;
  const Pub GU(P.gu);
  // the layer input and the router's partial logits complete (one wait): the
  // input's operand loads, then this claimer's own top-k and route, whose
  // loads share their round trip
  if (!wait_task(P, t, sm)) return;
  set_rows_batch(P, sm, 0, P.H, 0);
  __syncthreads();
  ATile<1, NCH> Ah0, Al0, Ah1, Al1;
  atile_load_bf16(Ah0, Pub(u_of(P, l, 0)), sm.row_off[0], 0, kh_chunks);
  atile_load_bf16(Al0, Pub(u_of(P, l, 1)), sm.row_off[0], 0, kh_chunks);
  atile_load_bf16(Ah1, Pub(u_of(P, l, 0)), sm.row_off[0], kh_chunks, kc);
  atile_load_bf16(Al1, Pub(u_of(P, l, 1)), sm.row_off[0], kh_chunks, kc);
  mark(sm, 0);
  route_build(P, l, sm, false);
  mark(sm, 1);
  const int n_items = __builtin_amdgcn_readfirstlane(sm.rt_hdr[1]);
  const int n_down = __builtin_amdgcn_readfirstlane(sm.rt_hdr[2]);
  const int64_t tot = pre(nt);
  const int lo = (int)(n_items * pre(sk) / tot), hi = (int)(n_items * pre(sk + 1) / tot);
  const int nd = wa == 0 ? nf : nt;  // down items: to the claimers with up/gate weight
  const int dlo = sk < nd ? (int)((int64_t)n_down * sk / nd) : 0;
  const int dhi = sk < nd ? (int)((int64_t)n_down * (sk + 1) / nd) : 0;
  const int DP = P.CB / 16, kcd = P.F / 32, dpe = P.down_items_per_expert;
  const size_t pstride_d = (size_t)kcd * 512;
  auto down_load = [&](WTile<4, NCHD>& w, int item, bool valid) {
    const int a = valid ? item / dpe : 0, cb = item % dpe;
    const int e = __builtin_amdgcn_readfirstlane(sm.rt_e[a]);
    wtile_load(w, P.wd + l * P.s_wd_l + (size_t)e * P.s_wd_e + (size_t)(cb * DP) * pstride_d, pstride_d,
               valid ? DP : 0, 0, kcd);
  };
  auto up_load = [&](WTile<2, NCH>& w, int id) {
    const bool valid = id < hi;
    const int a = valid ? id / upe : 0, r = id % upe;
    const int tt = r >> 1, kh = r & 1;
    const int e = __builtin_amdgcn_readfirstlane(sm.rt_e[a]);
    const int c0 = kh * kh_chunks;
    wtile_load(w, P.wgu + l * P.s_wgu_l + (size_t)e * P.s_wgu_e + (size_t)(2 * tt) * pstride, pstride,
               valid ? 2 : 0, c0, c0 + kh_chunks);
  };
  auto up_do = [&](const WTile<2, NCH>& w, int id) {
    const int a = id / upe, r = id % upe;
    const int tt = r >> 1, kh = r & 1;
    const int cnt = sm.rt_cnt[a];
    // this K half's operand (a bitwise blend: a select between the two tiles
    // would be turned into a dynamically indexed array in scratch)
    ATile<1, NCH> Hh, Hl;
    const uint32_t hi_half = 0u - (uint32_t)kh;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      Hh.a[0][i] = (Ah1.a[0][i] & hi_half) | (Ah0.a[0][i] & ~hi_half);
      Hl.a[0][i] = (Al1.a[0][i] & hi_half) | (Al0.a[0][i] & ~hi_half);
    }
    Acc<2, 1> acc;
    mfma_tiles(acc, w, Hh, Hl);
    reduce_tiles(acc, sm);
    // gu[slot][kh][gate|up][F] for the tokens routed to the expert: at most
    // 2 x 16 x 16 values, one per thread
    const int o = tid();
    if (o < 2 * cnt * 16) {
      const int which = o / (cnt * 16), rr = (o / 16) % cnt, nn = o % 16;
      const int slot = sm.rt_slot[a * B + rr], b = slot / K;
      GU.stf(((slot * 2 + kh) * 2 + which) * F + tt * 16 + nn, sm.out[which * 256 + b * 16 + nn] * sm.inv_rms[b]);
    }
  };
  {
    // UPD items in flight; a load past the share's end reads nothing (a zero
    // tile), so every iteration issues the same loads and the compiler waits
    // for exactly the item it computes next
    WTile<2, NCH> w[UPD];
#pragma unroll
    for (int k = 0; k < UPD; ++k) up_load(w[k], lo + k);
    for (int id = lo; id < hi; id += UPD) {
#pragma unroll
      for (int k = 0; k < UPD; ++k) {
        if (id + k < hi) up_do(w[k], id + k);
        up_load(w[k], id + k + UPD);
      }
    }
  }
  // this share's up/gate arrivals (one per item, on its expert's counter),
  // then the first down pair's weights
  sync_published();
  if (lo < hi) {
    const int a0 = lo / upe, a1 = (hi - 1) / upe;
    const int a = a0 + (int)tid();
    if (a <= a1) {
      const int n = min(hi, (a + 1) * upe) - max(lo, a * upe);
      __hip_atomic_fetch_add(&P.ctr[done_base + a], (uint32_t)n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // down items in groups of one or two blocks of one expert
  auto group_n = [&](int i) { return (i + 1 < dhi && (i + 1) % dpe != 0) ? 2 : 1; };
  WTile<4, NCHD> wd0, wd1;
  down_load(wd0, dlo, dlo < dhi);
  down_load(wd1, dlo + 1, dlo < dhi && group_n(dlo) == 2);
  mark(sm, 2);
  int staged = -1;
  for (int i = dlo; i < dhi;) {
    const int a = i / dpe, cb0 = i % dpe, ng = group_n(i);
    if (i > dlo) {
      down_load(wd0, i, true);
      down_load(wd1, i + 1, ng == 2);
    }
    down_pair<NCHD>(P, t, a, cb0, ng, wd0, wd1, a != staged, sm);
    staged = a;
    i += ng;
    if (error_seen(error_peek(P), sm)) return;
  }
  mark(sm, 3);
}

// Expert down over one column block for all tokens routed to expert slot a
// (megakernel post, section "Tasks": MOE_DOWN_DRAIN). Its weights (w) were
// loaded before this waits for that expert's up/gate items (section "What we
// have done differently": MoE down streams weights while up/gate still
// computes the hidden state it consumes). The contribution counts on the
// column block; the last one does the residual add.
// stage = false: the operand in LDS is the previous item's, of the same
// expert with at most 16 routed rows (already waited for and staged).
template <int MT, int NCH>
__device__ __forceinline__ void down_item(const mk_params& P, const mk_task& t, int a, int cb, const WTile<4, NCH>& w,
                                          Smem& sm, bool stage) {
  const int F = P.F, H = P.H, B = P.B;
  const int kc = F / 32;
  const int DP = P.CB / 16;
  const int cnt = sm.rt_cnt[a];
  const Pub DN(P.dn), GU(P.gu);
  stage = stage || cnt > 16;
  // the up/gate items may run in this same launch (kernel-per-op variant too)
  if (stage && !wait_one(P, t.a[1] + a, P.up_items_per_expert, sm, true)) return;
  // act = silu(g0 + g1) * (u0 + u1) per routed row, staged in LDS as the
  // split pair (16 rows at a time: hi in act[0, 16F), lo in act[16F, 32F))
  Acc<4, MT> acc;
#pragma unroll
  for (int pp = 0; pp < 4; ++pp)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc.c[pp][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int n = 16 * F;
    if (mt * 16 >= cnt) break;  // (uniform) no routed rows in this tile
    if (stage) stage_act(P, a, mt * 16, min(16, cnt - mt * 16), sm);
    const int wv = wave_id(), ln = lane_id();
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = wv + MK_WAVES * i;
      const int off = (ln & 15) * F + 32 * c + 8 * (ln >> 4);
      const u32x4_t ah = c < kc ? *(const u32x4_t*)(sm.act + off) : u32x4_t{0u, 0u, 0u, 0u};
      const u32x4_t al = c < kc ? *(const u32x4_t*)(sm.act + n + off) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        acc.c[pp][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, al),
                                                                __builtin_bit_cast(bf16x8_t, w.v[pp][i]),
                                                                acc.c[pp][mt], 0, 0, 0);
        acc.c[pp][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ah),
                                                                __builtin_bit_cast(bf16x8_t, w.v[pp][i]),
                                                                acc.c[pp][mt], 0, 0, 0);
      }
    }
    lds_sync();
  }
  reduce_tiles(acc, sm);
  for (int o = tid(); o < 4 * MT * 256; o += MK_WG_THREADS) {
    const int pp = o / (MT * 256), mt = (o / 256) % MT, m = (o / 16) % 16, nn = o % 16;
    const int row = mt * 16 + m;
    if (pp < DP && row < cnt) DN.stf(sm.rt_slot[a * B + row] * H + (cb * DP + pp) * 16 + nn, sm.out[o]);
  }
  block_arrive(P, t, t.a[4], cb, sm);
}

// The same with FP8 down codes in chunk pairs (pair p = wave + 8 i of the
// expert's K = F rows), converted to bf16 operands in registers; the staged
// operand carries the unit scales (stage_act with the expert's scale rows).
template <int MT, int NPR>
__device__ __forceinline__ void down_item(const mk_params& P, const mk_task& t, int a, int cb,
                                          const WTile8<4, NPR>& w, Smem& sm, bool stage) {
  const int F = P.F, H = P.H, B = P.B;
  const int kp = F / 64;
  const int DP = P.CB / 16;
  const int cnt = sm.rt_cnt[a];
  const Pub DN(P.dn);
  stage = stage || cnt > 16;
  if (stage && !wait_one(P, t.a[1] + a, P.up_items_per_expert, sm, true)) return;
  const int e = __builtin_amdgcn_readfirstlane(sm.rt_e[a]);
  const float* sc = P.fsc + t.layer * P.s_fsc_l + (size_t)e * P.s_fsc_e;
  Acc<4, MT> acc;
#pragma unroll
  for (int pp = 0; pp < 4; ++pp)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc.c[pp][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int n = 16 * F;
    if (mt * 16 >= cnt) break;  // (uniform) no routed rows in this tile
    if (stage) stage_act(P, a, mt * 16, min(16, cnt - mt * 16), sm, sc);
    const int wv = wave_id(), ln = lane_id();
#pragma unroll
    for (int i = 0; i < NPR; ++i) {
      const int p = wv + MK_WAVES * i;
      u32x4_t b[4][2];
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) e4m3x16_to_bf16(w.v[pp][i], b[pp][0], b[pp][1]);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = 2 * p + h;
        const int off = (ln & 15) * F + 32 * c + 8 * (ln >> 4);
        const u32x4_t ah = p < kp ? *(const u32x4_t*)(sm.act + off) : u32x4_t{0u, 0u, 0u, 0u};
        const u32x4_t al = p < kp ? *(const u32x4_t*)(sm.act + n + off) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          acc.c[pp][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, al),
                                                                  __builtin_bit_cast(bf16x8_t, b[pp][h]),
                                                                  acc.c[pp][mt], 0, 0, 0);
          acc.c[pp][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ah),
                                                                  __builtin_bit_cast(bf16x8_t, b[pp][h]),
                                                                  acc.c[pp][mt], 0, 0, 0);
        }
      }
    }
    lds_sync();
  }
  reduce_tiles(acc, sm);
  for (int o = tid(); o < 4 * MT * 256; o += MK_WG_THREADS) {
    const int pp = o / (MT * 256), mt = (o / 256) % MT, m = (o / 16) % 16, nn = o % 16;
    const int row = mt * 16 + m;
    if (pp < DP && row < cnt) DN.stf(sm.rt_slot[a * B + row] * H + (cb * DP + pp) * 16 + nn, sm.out[o]);
  }
  block_arrive(P, t, t.a[4], cb, sm);
}


// ------------------------------------------------------- fused MoE
// Batches of at most MK_FUSED_B tokens. An item is one 16-row slice s of an
// active expert's hidden layer: the slice's gate and up columns over the whole
// K (two K halves on the matrix cores), SiLU(gate) * up scaled by the routing
// weight of each token routed to the expert, then the slice's 16 rows of the
// down projection, accumulated per token over the claimer's items (megakernel
// post, section "Tasks": MOE_UPGATE_ACT and MOE_DOWN with the weighted sum of
// MOE_COMBINE; the hidden slice never leaves the compute unit, so there is
// no up/gate-to-down dependency between compute units). Each claimer stores
// one row per token its items saw; the residual tasks sum the rows.

// Claimer k's share [lo, hi) of n_items: claimers [0, nf) weigh 256, the
// others wa (of 256). The host schedules the same shares.
__device__ __forceinline__ void fused_share(int k, int nf, int nt, int wa, int n_items, int& lo, int& hi) {
  auto pre = [&](int j) -> int64_t { return j <= nf ? (int64_t)j * 256 : (int64_t)nf * 256 + (int64_t)(j - nf) * wa; };
  const int64_t tot = pre(nt);
  lo = (int)(n_items * pre(k) / tot);
  hi = (int)(n_items * pre(k + 1) / tot);
}

// Tokens (bit b) routed to the active experts of items [lo, hi) (S items per expert).
__device__ __forceinline__ uint32_t fused_tokens(const mk_params& P, const Smem& sm, int lo, int hi, int S) {
  uint32_t m = 0u;
  if (lo < hi)
    for (int a = lo / S; a <= (hi - 1) / S; ++a)
      for (int r = 0; r < sm.rt_cnt[a]; ++r) m |= 1u << (sm.rt_slot[a * P.B + r] / P.K);
  return m;
}

// Slice s (rows 16 s .. 16 s + 15) of a down projection [F x H] in the
// panel-tiled layout: in each of the H / 16 panels, one 512-byte half of
// chunk s / 2. Thread t takes piece t % 32 of that half (column t % 16, rows
// 8 ((t / 16) % 2) .. + 7 of the slice) in panels t / 32 + 16 j. An invalid
// slice reads nothing (zeros).
template <int NJ>
struct DTile {
  u32x4_t v[NJ];
};

template <int NJ>
__device__ __forceinline__ void dtile_load(DTile<NJ>& d, const uint16_t* base, size_t pstride, int npan, int s,
                                           bool valid) {
  const int t = tid();
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(base), (short)0, valid ? npan * (int)pstride * 2 : 0, 0x00020000);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int p = (t >> 5) + 16 * j;
    const int off = p < npan ? (p * (int)pstride + (s >> 1) * 512 + (s & 1) * 256) * 2 + (t & 31) * 16 : 0x7ffffff0;
    d.v[j] = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNT);
  }
}

// Activation operand from the layer input staged in LDS (xs: [MK_FUSED_B][H]
// bf16, one part of the split pair); rows at or beyond B are zero.
template <int NCH>
__device__ __forceinline__ void atile_lds(ATile<1, NCH>& A, const uint16_t* xs, int H, int B, int c0, int c1) {
  const int wv = wave_id(), ln = lane_id(), row = ln & 15;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = c0 + wv + MK_WAVES * i;
    A.a[0][i] = (c < c1 && row < B) ? *(const u32x4_t*)(xs + row * H + 32 * c + 8 * (ln >> 4)) : u32x4_t{0u, 0u, 0u, 0u};
  }
}

template <int NJ, int NCH, bool DENSE, bool FP8>
__device__ __forceinline__ void op_moe_fused(const mk_params& P, const mk_task& t, Smem& sm) {
  const int sk = t.b[0], nf = t.b[1], nt = t.b[2], wa = P.waits_enabled ? t.b[3] : 256;
  const int l = t.layer;
  const int F = P.F, H = P.H, B = P.B;
  const int S = F / 16;
  const int kc = H / 32, kh_chunks = kc / 2;
  const size_t pstride = (size_t)kc * 512, pstride_d = (size_t)(F / 32) * 512;
  // LDS: the layer input's split pair [2][MK_FUSED_B][H] (bf16), then the
  // current slice's weighted hidden values [MK_FUSED_B][16] (float)
  uint16_t* xs = sm.act;
  float* actf = reinterpret_cast<float*>(sm.act + 2 * MK_FUSED_B * MK_MAX_H);
  // the items' weights: an item past the share reads nothing; a dense
  // layer's one FFN is expert 0
  int lo = 0, hi = 0;
  auto expert_of = [&](int a) { return DENSE ? 0 : __builtin_amdgcn_readfirstlane(sm.rt_e[a]); };
  // (FP8: gate/up codes in chunk pairs, kh_pairs per K half; the down
  // slice's codes and the item's scales, a float4 (gate, up, down, 0) per
  // hidden unit, loaded by the threads that apply them)
  constexpr int NJ8 = MK_MAX_H / MK_WG_THREADS;
  const int kh_pairs = H / 128, pstride8 = (H / 64) * 1024;
  using WU = std::conditional_t<FP8, WTile8<2, NCH / 2>, WTile<2, NCH>>;
  using WD = std::conditional_t<FP8, DTile8<NJ8>, DTile<NJ>>;
  // (the scales of the item whose down tile was loaded last)
  float4 sc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto up_load = [&](WU& w, int id, int kh) {
    const bool valid = id < hi;
    const int a = valid ? id / S : 0, s = id % S;
    const int e = expert_of(a);
    if constexpr (FP8)
      wtile8_load(w, P.wgu8 + l * P.s_gu8_l + (size_t)e * P.s_gu8_e + (size_t)(2 * s) * pstride8, pstride8,
                  valid ? 2 : 0, kh * kh_pairs, (kh + 1) * kh_pairs);
    else
      wtile_load(w, P.wgu + l * P.s_wgu_l + (size_t)e * P.s_wgu_e + (size_t)(2 * s) * pstride, pstride,
                 valid ? 2 : 0, kh * kh_chunks, (kh + 1) * kh_chunks);
  };
  auto down_load = [&](WD& d, int id) {
    const bool valid = id < hi;
    const int a = valid ? id / S : 0, s = id % S;
    const int e = expert_of(a);
    if constexpr (FP8) {
      dtile8_load(d, P.wd8 + l * P.s_d8_l + (size_t)e * P.s_d8_e + (size_t)s * H * 16, H, valid);
      sc = valid && tid() < 16 * MK_FUSED_B
                    ? *(const float4*)(P.fsc + l * P.s_fsc_l + (size_t)e * P.s_fsc_e + 4 * (16 * s + (tid() & 15)))
                    : make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
      dtile_load(d, P.wd + l * P.s_wd_l + (size_t)e * P.s_wd_e, pstride_d, H / 16, s, valid);
    }
  };
  WU wu0, wu1;
  WD wdn;
  // A dense layer's FFN and this claimer's share of its slices are known
  // before the input is: the first slice's three weight units stream before
  // the wait (weight prefetch, megakernel post section "Where the speedup
  // comes from"). An expert's weights wait for the route.
  if constexpr (DENSE) {
    fused_share(sk, nf, nt, wa, S, lo, hi);
    up_load(wu0, lo, 0);
    up_load(wu1, lo, 1);
    down_load(wdn, lo);
  }
  // the layer input and the router's partial logits complete (one wait):
  // the input's loads, then this claimer's own top-k and route (whose loads
  // share the input's round trip), then the input into LDS
  // (tagged: only the input's counter; the router's partials are polled as
  // tagged words in the same round trip as the input's loads)
  if (!DENSE && P.tagged) {
    if (!wait_one(P, t.wait_ctr[0], t.wait_tgt[0], sm)) return;
  } else if (!wait_task(P, t, sm)) {
    return;
  }
  mark(sm, 0);
  {
    const Pub Uh(u_of(P, l, 0)), Ul(u_of(P, l, 1));
    const int n8 = B * H / 8;  // 8 bf16 per thread and load
    u32x4_t vh[MK_FUSED_B * MK_MAX_H / 8 / MK_WG_THREADS], vl[MK_FUSED_B * MK_MAX_H / 8 / MK_WG_THREADS];
#pragma unroll
    for (int k = 0; k < MK_FUSED_B * MK_MAX_H / 8 / MK_WG_THREADS; ++k) {
      const int i = tid() + k * MK_WG_THREADS;
      vh[k] = i < n8 ? Uh.ld16x8(8 * i) : u32x4_t{0u, 0u, 0u, 0u};
      vl[k] = i < n8 ? Ul.ld16x8(8 * i) : u32x4_t{0u, 0u, 0u, 0u};
    }
    if constexpr (DENSE) {
      route_trivial(P, l, sm, true);
    } else {
      // the active experts, then this claimer's share and its first item's
      // three weight units, then the rest of the route while they stream
      int n_active = 0;
      if (!route_rank(P, l, sm, false, n_active)) return;
      fused_share(sk, nf, nt, wa, n_active * S, lo, hi);
      up_load(wu0, lo, 0);
      up_load(wu1, lo, 1);
      down_load(wdn, lo);
      route_finish(P, l, sm, false, n_active);
    }
#pragma unroll
    for (int k = 0; k < MK_FUSED_B * MK_MAX_H / 8 / MK_WG_THREADS; ++k) {
      const int i = tid() + k * MK_WG_THREADS;
      if (i < n8) {
        *(u32x4_t*)(xs + 8 * i) = vh[k];
        *(u32x4_t*)(xs + MK_FUSED_B * MK_MAX_H + 8 * i) = vl[k];
      }
    }
    lds_sync();
  }
  const uint16_t* xh = xs;
  const uint16_t* xl = xs + MK_FUSED_B * MK_MAX_H;
  mark(sm, 1);
  constexpr int NA = FP8 ? NJ8 : NJ;
  float acc[NA][MK_FUSED_B];
#pragma unroll
  for (int j = 0; j < NA; ++j)
#pragma unroll
    for (int b = 0; b < MK_FUSED_B; ++b) acc[j][b] = 0.f;
  {
    // one item's three weight units in flight while the previous item's
    // compute: each unit is reissued for the next item as soon as it is used
    const int rh = (lane_id() >> 4) & 1;
    for (int id = lo; id < hi; ++id) {
      const int a = id / S;
      Acc<2, 1> ac;
      if constexpr (FP8) {
        {
          ATile<1, NCH> Ah, Al;
          atile_lds_pairs(Ah, xh, H, B, 0, kh_pairs);
          atile_lds_pairs(Al, xl, H, B, 0, kh_pairs);
          mfma_tiles8(ac, wu0, Ah, Al, false);
        }
        up_load(wu0, id + 1, 0);
        {
          ATile<1, NCH> Ah, Al;
          atile_lds_pairs(Ah, xh, H, B, kh_pairs, 2 * kh_pairs);
          atile_lds_pairs(Al, xl, H, B, kh_pairs, 2 * kh_pairs);
          mfma_tiles8(ac, wu1, Ah, Al, true);
        }
        up_load(wu1, id + 1, 1);
      } else {
        {
          ATile<1, NCH> Ah, Al;
          atile_lds(Ah, xh, H, B, 0, kh_chunks);
          atile_lds(Al, xl, H, B, 0, kh_chunks);
          mfma_tiles(ac, wu0, Ah, Al);
        }
        up_load(wu0, id + 1, 0);
        {
          ATile<1, NCH> Ah, Al;
          atile_lds(Ah, xh, H, B, kh_chunks, kc);
          atile_lds(Al, xl, H, B, kh_chunks, kc);
          mfma_tiles_add(ac, wu1, Ah, Al);
        }
        up_load(wu1, id + 1, 1);
      }
      reduce_tiles(ac, sm);
      // weighted SiLU(gate) * up of the slice for every token routed to the expert
      {
        // (the thread index tied to the item: its LDS addresses are then
        // formed here, not hoisted out of every loop and kept live)
        int o = tid();
        asm("" : "+v"(o) : "s"(id));
        if (o < MK_FUSED_B * 16) {
          const int b = o >> 4, r = o & 15;
          float v = 0.f;
          if (b < B) {
            int slot = -1;
            for (int rr = 0; rr < sm.rt_cnt[a]; ++rr) {
              const int s2 = sm.rt_slot[a * B + rr];
              if (s2 / P.K == b) slot = s2;
            }
            if (slot >= 0) {
              const float inv = sm.inv_rms[b];
              float g = sm.out[b * 16 + r] * inv, u = sm.out[256 + b * 16 + r] * inv;
              if constexpr (FP8) {
                g *= sc.x;
                u *= sc.y;
              }
              v = sm.tkw[slot] * (g / (1.0f + __expf(-g)) * u);
              if constexpr (FP8) v *= sc.z;
            }
          }
          actf[o] = v;
        }
      }
      __syncthreads();
      if constexpr (FP8) {
        // the slice's 16 down rows of columns t + 512 j, converted once and
        // applied to every token
#pragma unroll
        for (int j = 0; j < NJ8; ++j) {
          float wv[16];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const auto p0 = __builtin_amdgcn_cvt_pk_f32_fp8(wdn.v[j][k], false);
            const auto p1 = __builtin_amdgcn_cvt_pk_f32_fp8(wdn.v[j][k], true);
            wv[4 * k] = p0[0];
            wv[4 * k + 1] = p0[1];
            wv[4 * k + 2] = p1[0];
            wv[4 * k + 3] = p1[1];
          }
#pragma unroll
          for (int b = 0; b < MK_FUSED_B; ++b) {
            if (b < B) {
              float x = acc[j][b];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const float4 av = *(const float4*)(actf + b * 16 + 4 * q);
                x = fmaf(av.x, wv[4 * q], x);
                x = fmaf(av.y, wv[4 * q + 1], x);
                x = fmaf(av.z, wv[4 * q + 2], x);
                x = fmaf(av.w, wv[4 * q + 3], x);
              }
              acc[j][b] = x;
            }
          }
        }
      } else {
      // the slice's down rows: 8 of them per thread, one token at a time
#pragma unroll
      for (int b = 0; b < MK_FUSED_B; ++b) {
        if (b < B) {
          const float4 p = *(const float4*)(actf + b * 16 + 8 * rh);
          const float4 q = *(const float4*)(actf + b * 16 + 8 * rh + 4);
          const float x[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
#pragma unroll
          for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const uint32_t w2 = wdn.v[j][k];
              acc[j][b] = fmaf(x[2 * k + 1], __uint_as_float(w2 & 0xffff0000u),
                               fmaf(x[2 * k], __uint_as_float(w2 << 16), acc[j][b]));
            }
        }
      }
      }
      down_load(wdn, id + 1);
    }
  }
  mark(sm, 2);
  // rows 0-7 and 8-15 of each column, then this claimer's row of each token it saw
  const uint32_t seen = fused_tokens(P, sm, lo, hi, S);
  const Pub MP(P.mp);
  const int t0 = tid(), col = t0 & 15;
  const bool wr = ((t0 >> 4) & 1) == 0;
  if constexpr (FP8) {
#pragma unroll
    for (int j = 0; j < NJ8; ++j) {
      const int hh = t0 + MK_WG_THREADS * j;
#pragma unroll
      for (int b = 0; b < MK_FUSED_B; ++b)
        if (hh < H && b < B && ((seen >> b) & 1u)) MP.stf((sk * MK_FUSED_B + b) * H + hh, acc[j][b]);
    }
  } else
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int p = (t0 >> 5) + 16 * j;
#pragma unroll
    for (int b = 0; b < MK_FUSED_B; ++b) {
      const float v = sum16(acc[j][b]);
      if (wr && p < H / 16 && b < B && ((seen >> b) & 1u)) MP.stf((sk * MK_FUSED_B + b) * H + p * 16 + col, v);
    }
  }
  arrive_nr(P, t.sig_ctr[0]);
  mark(sm, 3);
}

// The published route of layer l into LDS (header, active experts, token counts, slots).
__device__ __forceinline__ void route_load(const mk_params& P, int l, Smem& sm) {
  const Pub R(route_of(P, l));
  const int E = P.E, B = P.B, i = tid();
  if (i < 4) sm.rt_hdr[i] = R.ldi(i);
  if (i < E) {
    sm.rt_e[i] = R.ldi(4 + i);
    sm.rt_cnt[i] = R.ldi(4 + E + i);
  }
  for (int k = i; k < E * B; k += MK_WG_THREADS) sm.rt_slot[k] = R.ldi(4 + 2 * E + k);
  __syncthreads();
}

// A dense layer's route into LDS: its one FFN is expert 0, every token is
// routed to it with weight 1 (slot b of token b); with `norm`, also layer
// l's sums of squares and 1/rms of every token (the FFN's input, written by
// the layer's mid residual).
__device__ __forceinline__ void route_trivial(const mk_params& P, int l, Smem& sm, bool norm) {
  const int B = P.B, i = tid();
  float sq[2] = {0.f, 0.f};
  if (norm) {
    const Pub S(ssq_of(P, l));
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int j = i + k * MK_WG_THREADS;
      sq[k] = j < B * P.NB ? S.ldf(j) : 0.f;
    }
  }
  if (i == 0) {
    sm.rt_hdr[0] = 1;
    sm.rt_hdr[1] = P.up_items_per_expert;
    sm.rt_hdr[2] = P.down_items_per_expert;
    sm.rt_hdr[3] = 0;
    sm.rt_e[0] = 0;
    sm.rt_cnt[0] = B;
  }
  if (i < B) {
    sm.rt_slot[i] = i;
    sm.tkw[i] = 1.0f;
  }
  if (norm) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int j = i + k * MK_WG_THREADS;
      if (j < B * P.NB) sm.ssq[j] = sq[k];
    }
  }
  lds_sync();
  if (norm) inv_rms_lds(P, sm);
  lds_sync();
}

// Residual add of column block cb once every fused MoE claimer and O
// projection of the layer has arrived: h += sum_g ao_g + the claimers' rows of
// each token (summed in claimer order), then the next layer's input and the
// block's sums of squares. Which claimers hold a row of which token follows
// from the route and the shares, worked out while the experts still run.
//   a[0] cb; b[1..3] as for the claimers; wait_ctr[0] every contribution,
//   wait_ctr[1] the route.
__device__ __forceinline__ void op_residual(const mk_params& P, const mk_task& t, Smem& sm) {
  const int l = t.layer, cb = t.a[0], mode = t.a[1];
  const int nf = t.b[1], nt = t.b[2], wa = P.waits_enabled ? t.b[3] : 256;
  const int H = P.H, CB = P.CB, B = P.B, n = B * CB;
  const int S = P.F / 16;
  const int i = tid();
  // the block's gain: the next layer's (the dense FFN's after attention)
  float h0 = 0.f, g0 = 0.f;
  if (i < n) {
    const int c = cb * CB + i % CB;
    g0 = bf2f(mode == MK_RES_DENSE_MID ? P.gamma2[(size_t)l * H + c] : P.gamma[(size_t)(l + 1) * H + c]);
  }
  if (mode == MK_RES_PARALLEL) {
    if (!wait_one(P, t.wait_ctr[1], t.wait_tgt[1], sm)) return;
    // The route is published by a task that waited for this layer's input,
    // so from here on the residual stream is the one this layer began with.
    // (Not before: nothing earlier on this unit need have waited for the
    // previous layer's residual tasks, which write it.)
    if (i < n) h0 = Pub(P.h).ldf((i / CB) * H + cb * CB + i % CB);
    route_load(P, l, sm);
  } else if (mode == MK_RES_DENSE_FFN) {
    route_trivial(P, l, sm, false);
  }
  // (claimer, token) rows, token-major, claimers ascending: per wave ballots
  // (none after a dense layer's attention)
  int* list = sm.rt_slot + 128 * MK_FUSED_B;  // past the slots of at most MK_FUSED_B tokens
  int* wcnt = sm.ired;                         // per wave, one token at a time
  const int n_items = mode == MK_RES_DENSE_MID ? 0 : sm.rt_hdr[0] * S;
  uint32_t mine = 0u;
  if (i < nt && mode != MK_RES_DENSE_MID) {
    int lo, hi;
    fused_share(i, nf, nt, wa, n_items, lo, hi);
    mine = fused_tokens(P, sm, lo, hi, S);
  }
  int* tb = sm.tb;
  if (i == 0) tb[0] = 0;
  for (int b = 0; b < B; ++b) {
    const bool has = (mine >> b) & 1u;
    const uint64_t bal = __ballot(has);
    if (lane_id() == 0) wcnt[wave_id()] = __popcll(bal);
    __syncthreads();
    int before = tb[b];
    for (int w = 0; w < wave_id(); ++w) before += wcnt[w];
    if (has) list[before + __popcll(bal & ((1ull << lane_id()) - 1ull))] = i;
    if (i == 0) {
      int tot = tb[b];
      for (int w = 0; w < MK_WAVES; ++w) tot += wcnt[w];
      tb[b + 1] = tot;
    }
    __syncthreads();
  }
  // every contribution has arrived
  if (!wait_one(P, t.wait_ctr[0], t.wait_tgt[0], sm)) return;
  mark(sm, 0);
  float av[MK_MAX_KVH];
  {
    const int b = i / CB, c = cb * CB + i % CB;
    if (mode != MK_RES_PARALLEL && i < n) h0 = Pub(P.h).ldf(b * H + c);
    const Pub ao(P.ao);
    const int ng = mode == MK_RES_DENSE_FFN ? 0 : P.KVH;  // the O projection's partials
#pragma unroll
    for (int g = 0; g < MK_MAX_KVH; ++g) av[g] = (i < n && g < ng) ? ao.ldf((g * B + b) * H + c) : 0.f;
  }
  // the rows: thread = (column quad cq, group gq); groups stride the list
  // (a row's NQ quads in adjacent lanes, so each load instruction reads whole
  // rows; the groups of a wave summed with a butterfly, then the 8 waves')
  const int NQ = CB / 4, NG = MK_WG_THREADS / NQ;
  const int cq = i % NQ, gq = i / NQ;
  // the rows through a resource over exactly the claimers' rows: a row past
  // the token's list reads past the end (zeros), so the loads carry no branch
  const __amdgpu_buffer_rsrc_t mr =
      __builtin_amdgcn_make_buffer_rsrc(P.mp, (short)0, nt * MK_FUSED_B * H * 4, 0x00020000);
  float4* red = reinterpret_cast<float4*>(sm.u.red);  // [MK_FUSED_B][MK_WAVES][NQ]
  for (int b = 0; b < B; ++b) {
    float4 s4 = make_float4(0.f, 0.f, 0.f, 0.f);
    const int p0 = tb[b], p1 = tb[b + 1];
    for (int p = p0 + gq; p < p1; p += 8 * NG) {
      u32x4_t x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int pu = p + u * NG;
        const int off = pu < p1 ? ((list[pu] * MK_FUSED_B + b) * H + cb * CB + 4 * cq) * 4 : 0x7ffffff0;
        x[u] = __builtin_amdgcn_raw_buffer_load_b128(mr, off, 0, kSC1);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        s4.x += __uint_as_float(x[u][0]);
        s4.y += __uint_as_float(x[u][1]);
        s4.z += __uint_as_float(x[u][2]);
        s4.w += __uint_as_float(x[u][3]);
      }
    }
    // (the wave's groups: lanes that differ in the bits above the quad index)
    s4.x = group_sum_above(s4.x, NQ);
    s4.y = group_sum_above(s4.y, NQ);
    s4.z = group_sum_above(s4.z, NQ);
    s4.w = group_sum_above(s4.w, NQ);
    if (lane_id() < NQ) red[(b * MK_WAVES + wave_id()) * NQ + cq] = s4;
  }
  __syncthreads();
  mark(sm, 1);
  float hv[MK_MAX_BATCH * 64 / MK_WG_THREADS] = {}, gv[MK_MAX_BATCH * 64 / MK_WG_THREADS] = {};
  if (i < n) {
    const int b = i / CB;
    const float* rf = reinterpret_cast<const float*>(red);
    float y = 0.f;
#pragma unroll
    for (int w = 0; w < MK_WAVES; ++w) y += rf[(b * MK_WAVES + w) * CB + i % CB];
    float a = 0.f;
#pragma unroll
    for (int g = 0; g < MK_MAX_KVH; ++g)
      if (g < P.KVH) a += av[g];
    hv[0] = (h0 + a) + y;
    gv[0] = g0;
  }
  __syncthreads();
  mark(sm, 2);
  // (a dense layer's FFN input goes to layer l's input buffers: every reader
  // of those, the layer's QKV tasks, has finished before its attention did)
  write_block_input(P, mode == MK_RES_DENSE_MID ? l : l + 1, cb, hv, gv, n, sm);
  mark(sm, 3);
  arrive_nr(P, t.sig_ctr[0]);
}

// ----------------------------------------------------------------- LM head
// LM head over a range of panels, two at a time with the next pair's weights
// streaming while the current pair computes; each task keeps every token's
// best logit (the lowest index on ties) and the task that completes the head
// picks the greedy tokens (tiny-vllm walkthrough, section "The remaining
// layers and logits": replace the running best only on a strictly greater
// value).
__device__ __forceinline__ void final_argmax(const mk_params& P, Smem& sm);

// Panels [p, p + np): the products, then (while the tiles reduce) the next
// panels' weights into the same registers, then the logits and the running
// best of every token.
template <int NP, int MT, int NCH>
__device__ __forceinline__ void lm_pair(const mk_params& P, WTile<NP, NCH>& w, const ATile<MT, NCH>& Ah,
                                        const ATile<MT, NCH>& Al, int p, int np, int p1, float& bv, int& bi,
                                        Smem& sm) {
  Acc<NP, MT> acc;
  mfma_tiles(acc, w, Ah, Al);
  const int kc = P.H / 32;
  const size_t pstride = (size_t)kc * 512;
  if (p + NP < p1) wtile_load(w, P.wlm + (size_t)(p + NP) * pstride, pstride, min(NP, p1 - p - NP), 0, kc);
  reduce_tiles(acc, sm);
  for (int o = tid(); o < NP * MT * 256; o += MK_WG_THREADS) {
    const int pp = o / (MT * 256), mt = (o / 256) % MT, m = (o / 16) % 16, nn = o % 16;
    const int b = mt * 16 + m;
    if (pp < np && b < P.B) P.logits[(size_t)b * P.V + (p + pp) * 16 + nn] = sm.out[o] * sm.inv_rms[b];
  }
  if ((int)tid() < P.B) {
    const int b = tid(), mt = b / 16, m = b % 16;
    const float inv = sm.inv_rms[b];
    for (int pp = 0; pp < np; ++pp)
      for (int nn = 0; nn < 16; ++nn) {
        const float v = sm.out[(pp * MT + mt) * 256 + m * 16 + nn] * inv;
        if (v > bv) {
          bv = v;
          bi = (p + pp) * 16 + nn;
        }
      }
  }
  __syncthreads();
}

// NP panels per step (two steps' weights in registers at a time).
template <int MT, int NCH, int NP>
__device__ __forceinline__ void op_lmhead(const mk_params& P, const mk_task& t, Smem& sm) {
  const int p0 = t.a[0], p1 = t.a[1], ord = t.a[2];
  const int kc = P.H / 32;
  const size_t pstride = (size_t)kc * 512;
  const int L = P.L;
  WTile<NP, NCH> w0;
  wtile_load(w0, P.wlm + (size_t)p0 * pstride, pstride, min(NP, p1 - p0), 0, kc);
  if (!wait_task(P, t, sm)) return;
  set_rows_batch(P, sm, 0, P.H, 0);
  __syncthreads();
  ATile<MT, NCH> Ah, Al;
  atile_load_bf16(Ah, Pub(u_of(P, L, 0)), sm.row_off[0], 0, kc);
  atile_load_bf16(Al, Pub(u_of(P, L, 1)), sm.row_off[0], 0, kc);
  load_inv_rms(P, L, sm);
  float bv = kNegInf;
  int bi = 0x7fffffff;
  for (int p = p0; p < p1; p += NP) lm_pair(P, w0, Ah, Al, p, min(NP, p1 - p), p1, bv, bi, sm);
  if ((int)tid() < P.B) {
    Pub(P.lm_val).stf(tid() * P.n_lm_tasks + ord, bv);
    Pub(P.lm_arg).sti(tid() * P.n_lm_tasks + ord, bi);
  }
  const int old = arrive(P, t.a[3], sm);
  if (old == P.n_lm_tasks - 1) final_argmax(P, sm);
}

// Greedy token of every sequence from the LM-head tasks' candidates; with
// MK_STEP_ADVANCE the token becomes the next step's input and the length grows.
__device__ __forceinline__ void final_argmax(const mk_params& P, Smem& sm) {
  const int n = P.n_lm_tasks;
  const Pub LV(P.lm_val), LA(P.lm_arg);
  const int wv = wave_id(), ln = lane_id();
  for (int b = wv; b < P.B; b += MK_WAVES) {
    float v = kNegInf;
    int ix = 0x7fffffff;
    for (int base = 0; base < n; base += 4 * 64) {
      float cv[4];
      int ci[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = base + u * 64 + ln;
        cv[u] = i < n ? LV.ldf(b * n + i) : kNegInf;
        ci[u] = i < n ? LA.ldi(b * n + i) : 0x7fffffff;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (cv[u] > v || (cv[u] == v && ci[u] < ix)) { v = cv[u]; ix = ci[u]; }
    }
    auto step = [&](float ov, int oi) {
      if (ov > v || (ov == v && oi < ix)) { v = ov; ix = oi; }
    };
    // (the pair steps: both lanes pick the better of the same two entries)
    auto pair_step = [&](float av, int ai, float bv, int bi) {
      const bool a_first = av > bv || (av == bv && ai < bi);
      v = a_first ? av : bv;
      ix = a_first ? ai : bi;
    };
    {
      float av, bv;
      int ai, bi;
      pair32(v, av, bv);
      pair32(ix, ai, bi);
      pair_step(av, ai, bv, bi);
      pair16(v, av, bv);
      pair16(ix, ai, bi);
      pair_step(av, ai, bv, bi);
    }
    step(xor_lane<8>(v), xor_lane<8>(ix));
    step(xor_lane<4>(v), xor_lane<4>(ix));
    step(xor_lane<2>(v), xor_lane<2>(ix));
    step(xor_lane<1>(v), xor_lane<1>(ix));
    if (ln == 0) {
      if (ix == 0x7fffffff) {
        // no logit of the row compares greater than -inf (all NaN or -inf):
        // there is no greedy token, and the step reports it
        raise_error(P, MK_DEVERR_FAULT, 6000 + b, 0u);
      } else {
        if (P.next_tokens) P.next_tokens[b] = ix;
        if (P.flags & 1u) {
          P.tokens[b] = ix;
          P.seq_lens[b] = P.seq_lens[b] + 1;
        }
      }
    }
  }
}

// --------------------------------------------------------------- dispatch

template <int D, int MT, bool FP8>
__device__ __forceinline__ void run_task_mt(const mk_params& P, const mk_task& t, Smem& sm) {
  switch (t.op) {
    // chunks per wave: K / 32 / MK_WAVES for the largest K of each op
    // (hidden 2048, group width 1024, K half 1024, expert width 768)
    case MK_OP_EMBED: op_embed(P, t, sm); break;
    case MK_OP_QKV: op_qkv<MT, 64 / MK_WAVES>(P, t, sm); break;
    case MK_OP_ATTN: op_attn<D>(P, t, sm); break;
    case MK_OP_OPROJ:
      if (MT == 1 && t.b[1] == 1)  // batches up to MK_FUSED_B: merges the splits itself
        op_oproj<D, 1, 32 / MK_WAVES, 8, true>(P, t, sm);
      else
        op_oproj<D, MT, 32 / MK_WAVES, 4, false>(P, t, sm);
      break;
    case MK_OP_ROUTER: op_router<MT, 32 / MK_WAVES>(P, t, sm); break;
    case MK_OP_MOE_UP:
      // at most 16 tokens: fixed shares (b[2], the claimer count, is set);
      // above: claiming, each item's routed rows
      // (FP8 feed-forward weights: claiming at every batch above MK_FUSED_B)
      if constexpr (FP8)
        op_moe_gather<32 / MK_WAVES, 2, 24 / MK_WAVES, true, MT>(P, t, sm);
      else if constexpr (MT == 1)
        op_moe_static<32 / MK_WAVES, 24 / MK_WAVES, 4>(P, t, sm);
      else
        op_moe_gather<32 / MK_WAVES, 2, 24 / MK_WAVES, false, MT>(P, t, sm);
      break;
    case MK_OP_MOE_FUSED:
      // (a dense layer's FFN has its own instance: its weight prefetch before
      // the wait keeps tiles live there, which the experts' instance does not)
      if (MT == 1) {
        if (P.dense)
          op_moe_fused<2048 / 256, 32 / MK_WAVES, true, FP8>(P, t, sm);
        else
          op_moe_fused<2048 / 256, 32 / MK_WAVES, false, FP8>(P, t, sm);
      }
      break;
    case MK_OP_RESIDUAL:
      if (MT == 1) op_residual(P, t, sm);
      break;
    case MK_OP_LMHEAD: op_lmhead<MT, 64 / MK_WAVES, MT == 1 ? 2 : 1>(P, t, sm); break;
    default: wait_task(P, t, sm); break;
  }
}

}  // namespace

// The interpreter: workgroup i runs tasks [task_off[i], task_off[i+1]).
// MT: row tiles of 16 tokens (1 for batch <= 16, 2 for batch <= 32).
template <int D, int MT, bool FP8>
__global__ __launch_bounds__(MK_WG_THREADS, MK_WGS_PER_CU) void mk_interp(mk_params Pk) {
  __shared__ Smem sm;
  const mk_params& P = Pk;
  if (tid() == 0) sm.t_mark[0] = sm.t_mark[1] = sm.t_mark[2] = sm.t_mark[3] = 0;
  if (P.ctr_clear) {
    for (int i = blockIdx.x * MK_WG_THREADS + tid(); i < P.n_ctr; i += gridDim.x * MK_WG_THREADS)
      P.ctr_clear[i] = 0u;
  }
  __syncthreads();
  const int beg = P.task_off[blockIdx.x], end = P.task_off[blockIdx.x + 1];
  for (int i = beg; i < end; ++i) {
#if defined(__HIP_DEVICE_COMPILE__)
    // the descriptor through a constant-address-space pointer: its fields are
    // then read with scalar loads, batched, instead of one vector load per
    // field on the way into each wait
    typedef const __attribute__((address_space(4))) mk_task* ktask_ptr;
    const mk_task& t = *(const mk_task*)((ktask_ptr)P.tasks + i);
#else
    const mk_task& t = P.tasks[i];
#endif
    const uint32_t t0 = (uint32_t)__builtin_amdgcn_s_memrealtime();
    if (tid() == 0) {
      sm.t_mark[0] = sm.t_mark[1] = sm.t_mark[2] = sm.t_mark[3] = 0;
      sm.t_waited = t0;  // a task without waits
    }
    // The parameter block through an opaque copy of its (constant address
    // space) pointer per task: parameter fields are then loaded inside each op
    // with scalar loads instead of being hoisted out of the task loop and held
    // in registers across every op.
#if defined(__HIP_DEVICE_COMPILE__)
    typedef const __attribute__((address_space(4))) mk_params* kparams_ptr;
    kparams_ptr Pt = (kparams_ptr)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(Pt));
    run_task_mt<D, MT, FP8>(*(const mk_params*)Pt, t, sm);
#else
    run_task_mt<D, MT, FP8>(P, t, sm);
#endif
    // (LDS only: a task's stores need no draining here; every hand-off
    // through a counter drains before its arrival, and tagged words carry
    // their own readiness)
    lds_sync();
    if (P.trace && tid() == 0) {
      // per-task timestamps (100 MHz device clock): start, waits satisfied,
      // op-defined marks, end
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

template __global__ void mk_interp<64, 1, false>(mk_params);
template __global__ void mk_interp<64, 2, false>(mk_params);
template __global__ void mk_interp<128, 1, false>(mk_params);
template __global__ void mk_interp<128, 2, false>(mk_params);
// FP8 feed-forward weights
template __global__ void mk_interp<64, 1, true>(mk_params);
template __global__ void mk_interp<64, 2, true>(mk_params);
template __global__ void mk_interp<128, 1, true>(mk_params);
template __global__ void mk_interp<128, 2, true>(mk_params);

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
  for (int idx = tid(); idx < 32 * (width / 8); idx += 256) {
    const int row = idx / (width / 8), c8 = idx % (width / 8);
    const uint4 v = *(const uint4*)(s + (size_t)(32 * c + row) * ld + n0 + c8 * 8);
    *(uint4*)&tile[row][c8 * 8] = v;
  }
  __syncthreads();
  const int npan = width / 16;
  for (int idx = tid(); idx < npan * 64; idx += 256) {
    const int j = idx / 64, l = idx % 64;
    uint16_t tmp[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) tmp[i] = tile[8 * (l >> 4) + i][16 * j + (l & 15)];
    const int pj = dst0 + (n0 / 16 + j) * dstep;
    *(uint4*)(d + ((size_t)pj * kc + c) * 512 + l * 8) = *(uint4*)tmp;
  }
}

// FP8 codes of a [K x N] matrix (canonical row-major, bytes) -> panels of K / 64
// chunk pairs of 1 KB (the layout of the gate/up panels below, for any
// matrix): source panel j to destination panel dst0 + j * dstep; z strides
// both sides. One thread per 16-byte lane unit.
extern "C" __global__ __launch_bounds__(256) void mk_repack_fp8_panels(const uint8_t* src, uint8_t* dst, int K, int N,
                                                                       int dst0, int dstep, int nz,
                                                                       size_t src_zstride, size_t dst_zstride) {
  const int npair = K / 64, npan = N / 16;
  const size_t n = (size_t)nz * npan * npair * 64;
  for (size_t u = (size_t)blockIdx.x * 256 + threadIdx.x; u < n; u += (size_t)gridDim.x * 256) {
    const int l = (int)(u % 64), p = (int)((u / 64) % npair);
    const int j = (int)((u / ((size_t)64 * npair)) % npan);
    const int z = (int)(u / ((size_t)64 * npair * npan));
    const uint8_t* s = src + z * src_zstride;
    const int col = 16 * j + (l & 15);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const int row = 64 * p + (b >= 8 ? 32 : 0) + 8 * (l >> 4) + (b & 7);
      w[b >> 2] |= (uint32_t)s[(size_t)row * N + col] << (8 * (b & 3));
    }
    const int pj = dst0 + j * dstep;
    *(u32x4_t*)(dst + z * dst_zstride + ((size_t)pj * npair + p) * 1024 + l * 16) = u32x4_t{w[0], w[1], w[2], w[3]};
  }
}

// FP8 down codes: canonical wd [E][F][H] -> per expert [F / 16][H][16]: the
// 16 codes of rows 16 s .. 16 s + 15 of column h contiguous. One thread per
// (expert, slice, column).
extern "C" __global__ __launch_bounds__(256) void mk_repack_fp8_d(const uint8_t* wd, uint8_t* dst, int F, int H,
                                                                  int E) {
  const int S = F / 16;
  const size_t n = (size_t)E * S * H;
  for (size_t u = (size_t)blockIdx.x * 256 + threadIdx.x; u < n; u += (size_t)gridDim.x * 256) {
    const int h = (int)(u % H), sl = (int)((u / H) % S), e = (int)(u / ((size_t)H * S));
    const uint8_t* src = wd + (size_t)e * F * H + (size_t)(16 * sl) * H + h;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i >> 2] |= (uint32_t)src[(size_t)i * H] << (8 * (i & 3));
    *(u32x4_t*)(dst + u * 16) = u32x4_t{w[0], w[1], w[2], w[3]};
  }
}

// The three per-hidden-unit scale vectors as one float4 per unit (gate, up, down, 0).
extern "C" __global__ __launch_bounds__(256) void mk_pack_scales(const float* sg, const float* su, const float* sd,
                                                                 float* dst, int n) {
  for (int i = blockIdx.x * 256 + (int)threadIdx.x; i < n; i += gridDim.x * 256)
    *(float4*)(dst + 4 * (size_t)i) = make_float4(sg[i], su[i], sd[i], 0.f);
}

// ----------------------------------------------- static scratch (no allocation)
// The per-step scratch of mk_decode_step_noalloc: activations, partials,
// routing, counters and the error word of one step, in one file-scope device
// array (each device the library runs on holds its own copy until the
// process ends). In host code `scratch` names a host-side stand-in, never the
// device memory: host code uses only the address hipGetSymbolAddress gives
// for the current device (mk_static_scratch).
static __device__ __align__(256) unsigned char scratch[MK_STATIC_SCRATCH_BYTES];

// Zero n words (the counters of a step that must start at zero): a kernel, not
// a memset, so a caller may capture it in a graph.
extern "C" __global__ __launch_bounds__(256) void mk_zero_words(uint32_t* p, int n) {
  for (int i = blockIdx.x * 256 + (int)threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

// Fill n words with a pattern, word i taking lo (even i) or hi (odd i): the
// debug poison of the step's scratch (NaN for values, an impossible tag for
// tagged words).
extern "C" __global__ __launch_bounds__(256) void mk_fill_words(uint32_t* p, int n, uint32_t lo, uint32_t hi) {
  for (int i = blockIdx.x * 256 + (int)threadIdx.x; i < n; i += gridDim.x * 256) p[i] = (i & 1) ? hi : lo;
}

// The streaming-read ceiling, a diagnostic beside the megakernel's figures:
// each workgroup (two per compute unit, 512 threads) reads one contiguous
// range of the n16 16-byte words, 8 KB per round (consecutive lanes on
// consecutive words) with eight rounds' nontemporal loads in flight, as the
// weight streams of the decode step do. The words are folded into one value
// per thread that is stored only if it equals a constant the data never
// makes, so no load can be dropped and nothing is written. (The word has
// external linkage, so the store, and with it the loads, cannot be proven
// dead.)
__device__ uint32_t mk_stream_sink;

extern "C" __global__ __launch_bounds__(512) void mk_stream_read_words(const u32x4_t* p, size_t n16) {
  constexpr int U = 8;
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t lo = per * blockIdx.x, hi = lo + per < n16 ? lo + per : n16;
  size_t i = lo + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * 512 < hi; i += U * 512) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * 512);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < hi; i += 512) {
    const u32x4_t a = __builtin_nontemporal_load(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9e3779b9u) mk_stream_sink = acc;
}

// Cross-XCD message passing with the step's own primitives (a litmus test of
// the protocol every hand-off between compute units uses). Pair p is
// workgroups 2p (producer) and 2p + 1 (consumer), which the dispatcher places
// on different XCDs. For rounds r = 1..R the producer waits until the
// consumer has acknowledged round r - 1, writes a 16-word message holding r,
// drains its stores and increments the pair's flag (as a task does before it
// signals); the consumer polls the flag until it reaches r, reads the message
// and counts words below r (stale reads), then acknowledges. With coherent =
// 0 the message is written and read with plain accesses instead (the
// contrast). Every wait gives up after limit_ticks (100 MHz) and is counted;
// a pair stops at its first timeout or stale read, so the kernel always ends.
// result[2p] stale reads, result[2p + 1] timeouts. With coherent = 2 the
// message is the tagged words of the step's small hand-offs instead.
__device__ __forceinline__ bool litmus_wait(const uint32_t* f, uint32_t want, int64_t limit) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (ld_relaxed(f) < want) {
    __builtin_amdgcn_s_sleep(1);
    if ((int64_t)(__builtin_amdgcn_s_memrealtime() - t0) > limit) return false;
  }
  return true;
}

extern "C" __global__ __launch_bounds__(64) void mk_litmus_mp(uint32_t* msg, uint32_t* flag, uint32_t* ack,
                                                              uint32_t* result, int rounds, int coherent,
                                                              int64_t limit) {
  const int p = blockIdx.x >> 1, ln = threadIdx.x;
  const bool producer = (blockIdx.x & 1) == 0;
  uint32_t* m = msg + p * 64;  // 256 bytes per pair: its own lines
  const Pub M(m);
  __shared__ int stop;
  if (ln == 0) stop = 0;
  __syncthreads();
  uint32_t stale = 0, timeouts = 0;
  // tagged (coherent = 2): the message is 16 tagged words (value, round) that
  // the consumer polls itself, with no drain or flag on the producer's side;
  // a word whose value is not the one written with its tag counts as stale
  auto value_of = [](int r, int i) { return (uint32_t)r * 0x9E3779B1u + (uint32_t)i * 0x85EBCA77u; };
  for (int r = 1; r <= rounds && coherent == 2; ++r) {
    if (producer) {
      if (ln == 0 && !litmus_wait(ack + p, (uint32_t)(r - 1), limit)) stop = 1;
      __syncthreads();
      if (stop) {
        timeouts += ln == 0;
        break;
      }
      if (ln < 16) M.st_tagged(ln, value_of(r, ln), (uint32_t)r);
    } else {
      bool bad = false;
      if (ln < 8) {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        u32x4_t v = M.ld_tagged2(2 * ln);
        while (v[1] != (uint32_t)r || v[3] != (uint32_t)r) {
          if ((int64_t)(__builtin_amdgcn_s_memrealtime() - t0) > limit) {
            stop = 1;
            break;
          }
          v = M.ld_tagged2(2 * ln);
        }
        bad = !stop && (v[0] != value_of(r, 2 * ln) || v[2] != value_of(r, 2 * ln + 1));
      }
      __syncthreads();
      if (stop) {
        timeouts += ln == 0;
        break;
      }
      const uint64_t ballot = __ballot(bad);
      if (ballot) {
        stale += ln == 0 ? (uint32_t)__popcll(ballot) : 0u;
        if (ln == 0) stop = 1;
      }
      __syncthreads();
      if (ln == 0) __hip_atomic_fetch_add(ack + p, stop ? (1u << 30) : 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (stop) break;
    }
  }
  for (int r = 1; r <= rounds && coherent != 2; ++r) {
    if (producer) {
      if (ln == 0 && !litmus_wait(ack + p, (uint32_t)(r - 1), limit)) stop = 1;
      __syncthreads();
      if (stop) {
        timeouts += ln == 0;
        break;
      }
      if (ln < 16) {
        if (coherent)
          M.sti(ln, r);
        else
          m[ln] = (uint32_t)r;
      }
      drain_memory();
      __syncthreads();
      if (ln == 0) __hip_atomic_fetch_add(flag + p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      if (ln == 0 && !litmus_wait(flag + p, (uint32_t)r, limit)) stop = 1;
      __syncthreads();
      if (stop) {
        timeouts += ln == 0;
        break;
      }
      uint32_t v = 0;
      if (ln < 16) v = coherent ? (uint32_t)M.ldi(ln) : *(volatile uint32_t*)(m + ln);
      const bool bad = ln < 16 && v < (uint32_t)r;
      const uint64_t ballot = __ballot(bad);
      if (ballot) {
        stale += ln == 0 ? (uint32_t)__popcll(ballot) : 0u;
        if (ln == 0) stop = 1;
      }
      drain_memory();
      __syncthreads();
      // (stopping: the acknowledgement runs ahead of every later round, so
      // the producer finishes its rounds without waiting)
      if (ln == 0) __hip_atomic_fetch_add(ack + p, stop ? (1u << 30) : 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (stop) break;
    }
  }
  if (ln == 0 && !producer) result[2 * p] = stale;
  if (ln == 0) __hip_atomic_fetch_add(result + 2 * p + 1, timeouts, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------ host launch
#include <mutex>

#include "mk_launch.h"

hipError_t mk_static_scratch(int device, void** ptr) {
  static std::mutex mu;
  static void* addr[MK_MAX_DEVICES] = {};
  if (device < 0 || device >= MK_MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (cur != device) hipSetDevice(cur);
    if (e != hipSuccess) return e;
    addr[device] = a;
  }
  *ptr = addr[device];
  return hipSuccess;
}

hipError_t mk_launch_litmus(uint32_t* msg, uint32_t* flag, uint32_t* ack, uint32_t* result, int pairs, int rounds,
                            int coherent, int64_t limit, hipStream_t stream) {
  hipLaunchKernelGGL(mk_litmus_mp, dim3(2 * pairs), dim3(64), 0, stream, msg, flag, ack, result, rounds, coherent,
                     limit);
  return hipGetLastError();
}

hipError_t mk_launch_stream_read(const void* p, size_t n16, hipStream_t stream) {
  hipLaunchKernelGGL(mk_stream_read_words, dim3(512), dim3(512), 0, stream, (const u32x4_t*)p, n16);
  return hipGetLastError();
}

hipError_t mk_launch_fill(uint32_t* p, int n, uint32_t lo, uint32_t hi, hipStream_t stream) {
  const int grid = n <= 0 ? 1 : (n + 255) / 256 < 256 ? (n + 255) / 256 : 256;
  hipLaunchKernelGGL(mk_fill_words, dim3(grid), dim3(256), 0, stream, p, n, lo, hi);
  return hipGetLastError();
}

hipError_t mk_launch_zero(uint32_t* p, int n, hipStream_t stream) {
  const int grid = n <= 0 ? 1 : (n + 255) / 256 < 64 ? (n + 255) / 256 : 64;
  hipLaunchKernelGGL(mk_zero_words, dim3(grid), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

static const void* interp_fn(int head_dim, int mt, bool fp8 = false) {
  if (fp8 && head_dim == 64) return mt == 1 ? (const void*)mk_interp<64, 1, true> : (const void*)mk_interp<64, 2, true>;
  if (fp8) return mt == 1 ? (const void*)mk_interp<128, 1, true> : (const void*)mk_interp<128, 2, true>;
  if (head_dim == 64) return mt == 1 ? (const void*)mk_interp<64, 1, false> : (const void*)mk_interp<64, 2, false>;
  return mt == 1 ? (const void*)mk_interp<128, 1, false> : (const void*)mk_interp<128, 2, false>;
}

hipError_t mk_launch_interp(const mk_params& P, int head_dim, int grid, bool cooperative, hipStream_t stream) {
  const void* fn = interp_fn(head_dim, P.B > 16 ? 2 : 1, P.ffn_fp8 != 0);
  void* args[] = {(void*)&P};
  if (cooperative)
    return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(MK_WG_THREADS), args, 0, stream);
  return hipLaunchKernel(fn, dim3(grid), dim3(MK_WG_THREADS), args, 0, stream);
}

hipError_t mk_launch_repack_fp8_panels(const uint8_t* src, uint8_t* dst, int K, int N, int dst0, int dstep, int nz,
                                       size_t src_zstride, size_t dst_zstride, hipStream_t stream) {
  hipLaunchKernelGGL(mk_repack_fp8_panels, dim3(4096), dim3(256), 0, stream, src, dst, K, N, dst0, dstep, nz,
                     src_zstride, dst_zstride);
  return hipGetLastError();
}

hipError_t mk_launch_repack_fp8_d(const uint8_t* wd, uint8_t* dst, int F, int H, int E, hipStream_t stream) {
  hipLaunchKernelGGL(mk_repack_fp8_d, dim3(4096), dim3(256), 0, stream, wd, dst, F, H, E);
  return hipGetLastError();
}

hipError_t mk_launch_pack_scales(const float* sg, const float* su, const float* sd, float* dst, int n,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(mk_pack_scales, dim3(256), dim3(256), 0, stream, sg, su, sd, dst, n);
  return hipGetLastError();
}

hipError_t mk_launch_repack(const uint16_t* src, uint16_t* dst, int K, int N, int ld, int dst0, int dstep,
                            int nz, size_t src_zstride, size_t dst_zstride, hipStream_t stream) {
  dim3 grid(K / 32, (N + 511) / 512, nz);
  hipLaunchKernelGGL(mk_repack_panels, grid, dim3(256), 0, stream, src, dst, K, N, ld, dst0, dstep, src_zstride,
                     dst_zstride);
  return hipGetLastError();
}

// Resident workgroups per compute unit of the interpreter (the smaller of the
// two row-tile variants).
hipError_t mk_interp_occupancy(int head_dim, int* blocks_per_cu) {
  int a = 0, b = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, interp_fn(head_dim, 1), MK_WG_THREADS, 0);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, interp_fn(head_dim, 2), MK_WG_THREADS, 0);
  if (e != hipSuccess) return e;
  for (int mt = 1; mt <= 2; ++mt) {
    int c = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&c, interp_fn(head_dim, mt, true), MK_WG_THREADS, 0);
    if (e != hipSuccess) return e;
    if (c < b) b = c;
  }
  *blocks_per_cu = a < b ? a : b;
  return e;
}
