// mk_internal.h - task descriptor, opcodes and kernel parameters shared by the
// host scheduler (mk_host.cpp) and the device interpreter (mk_device.hip).
//
// A task is one tile of one operation, described by 32 int32 fields (Cohere's
// North Mini Code megakernel post, section "The task descriptor": field 0 the
// opcode, then op-specific fields, the counters to wait on with their target
// counts, and the counter to signal). The fields are read with scalar loads
// because every lane of a workgroup runs the same task.
#pragma once
#include <stddef.h>
#include <stdint.h>

// One workgroup of 8 wave64s stays resident per compute unit and walks its
// task list (MK_WGS_PER_CU = 2 with 256 threads gives two independent lists
// per compute unit instead; measured slower: the dependent chain of a layer
// is latency-bound and a half-size workgroup takes twice as long per task).
#define MK_WG_THREADS 512
#define MK_WAVES (MK_WG_THREADS / 64)
#define MK_WGS_PER_CU 1
#define MK_MAX_CUS 1024
#define MK_MAX_TOPK 8
#define MK_MAX_KVH 8    // kv heads
#define MK_MAX_RKS 4    // router K splits
#define MK_MAX_F 768    // expert width
#define MK_MAX_H 2048   // hidden size
#define MK_MAX_BATCH 32
// Attention combine: split partials in flight per thread (16-byte loads)
#define MK_COMB_SB 16 // sequences per step (two row tiles of 16)
#define MK_UP_BATCH_MAX 4  // expert up/gate items claimed together
// Batches up to this size run the fused MoE: each claimer takes 16-row
// slices of the active experts' hidden layer through up/gate, SiLU and down,
// and stores one partial output row per token it saw; residual tasks sum them.
#define MK_FUSED_B 4
#define MK_MAX_DENSE_F 8192 // widest dense FFN
#define MK_TASK_INTS 32
// Static scratch of the allocation-free step: its size bounds the per-step
// scratch (and counters) of the models it accepts; the full-size model needs
// about 55 MB at batch 32 with 16K contexts.
#define MK_STATIC_SCRATCH_BYTES (64u << 20)
#define MK_MAX_DEVICES 64

// Opcodes. The post names sixteen opcodes for its model family; the ones
// below cover it. A dense layer's FFN (FFN_UPGATE_ACT, FFN_DOWN) runs as the
// fused claimer over its one FFN (MOE_FUSED with a fixed route). MOE_GATHER
// is folded into the expert up/gate task (it reads the routed token rows
// directly), MOE_COMBINE into
// the residual + RMSNorm step (it sums each token's k expert outputs in rank
// order while forming the residual), ROUTER_TOPK and ROUTE_FINALIZE into the
// last router task, ATTN_COMBINE into the last attention split, and the
// residual + RMSNorm itself into the last contribution to each column block.
enum mk_opcode : int32_t {
  MK_OP_NOP = 0,
  MK_OP_EMBED = 1,        // embedding rows of one column block: layer 0's input
  MK_OP_QKV = 2,          // QKV panels + RoPE + paged KV append
  MK_OP_ATTN = 3,         // split-KV partial attention (+ combine when last)
  MK_OP_RESIDUAL = 4,     // residual + MoE combine of one column block, the next layer's input (fused MoE;
                          // for a dense layer also the mid point: h + attention, the FFN's input)
  MK_OP_OPROJ = 5,        // O projection, split-K by kv group, one column block (+ residual when last)
  MK_OP_ROUTER = 6,       // router logits over a K range (+ top-k / finalize when last)
  MK_OP_MOE_UP = 8,       // MoE claimer: (expert, gate/up panel pair, K half) items, then
                          // (expert, column block) down items (+ residual when last)
  MK_OP_MOE_FUSED = 9,    // MoE claimer, small batches: (expert, 16-row hidden slice) items through
                          // up/gate, SiLU and down, one partial output row per token
  MK_OP_LMHEAD = 10,      // LM head panels + argmax candidate (+ greedy token when last)
  MK_OP_COUNT = 11
};

// Residual modes (a[1] of MK_OP_RESIDUAL): a parallel layer's end (O
// projection partials and the fused MoE claimers' rows; the next layer's
// input), a dense layer's mid point (O projection partials; the FFN's input
// with gamma2), a dense layer's end (the FFN claimers' rows; the next
// layer's input).
#define MK_RES_PARALLEL 0
#define MK_RES_DENSE_MID 1
#define MK_RES_DENSE_FFN 2

struct mk_task {
  int32_t op;
  int32_t layer;
  int32_t a[6];           // op arguments (see the op bodies)
  int32_t wait_ctr[3];    // counter index or -1
  int32_t wait_tgt[3];    // wait until counter >= target
  int32_t sig_ctr[2];     // counters incremented once when the task is done, or -1
  int32_t b[4];           // more op arguments (see the op bodies)
  int32_t pad[12];
};
static_assert(sizeof(mk_task) == MK_TASK_INTS * 4, "descriptor is 32 int32");

// Route scratch (int32), rebuilt per layer by the last router task:
//   [0] n_active experts, [1] n_up_items, [2] n_down_items, [3] unused
//   [4 .. 4+E)           active expert ids, ascending
//   [4+E .. 4+2E)        tokens routed to each active expert
//   [4+2E .. 4+2E+E*B)   per active expert: slots b*k + j routed to it, ascending b
#define MK_ROUTE_INTS(E, B) (4 + 2 * (E) + (E) * (B))

// Device error word: [0] code (0 none, 5 timeout, 6 fault), [1] detail, [2] value, [3] cu
#define MK_DEVERR_TIMEOUT 5
#define MK_DEVERR_FAULT 6

struct mk_params {
  // shape
  int32_t H, QH, KVH, D, G, E, K, F, V, L, PS, window, full_every;
  float eps;
  float attn_scale;
  int32_t B, mpps, n_pages, max_seq;
  int32_t up_items_per_expert;   // 2 * F / 16 (gate/up panel pairs x K halves)
  int32_t down_items_per_expert; // NB (column blocks)
  int32_t CB, NB;                // residual column block width (multiple of 16, <= 64) and count H / CB
  int32_t n_router_tasks, router_ks; // router tasks, and the K splits among them
  int32_t max_splits;            // attention partial slots per (sequence, group)
  int32_t n_lm_tasks;            // LM-head tasks (argmax candidates per sequence)
  int32_t e_pad;                 // router columns, padded to a multiple of 16
  // packed weights (bf16 bit patterns)
  const uint16_t* emb;           // [V][H] row-major
  const uint16_t* gamma;         // [L+1][H]
  const uint16_t* gamma2;        // dense models: [L][H] the FFN's norm gains
  int32_t dense;                 // 1: sequential dense layers (attention, then the FFN)
  const uint16_t* wqkv; size_t s_wqkv;      // per layer: panel-tiled [H x QKV]
  const uint16_t* wo; size_t s_wo;          // per layer: panel-tiled [QH*D x H]
  const uint16_t* wr; size_t s_wr;          // per layer: panel-tiled [H x e_pad]
  const uint16_t* wgu; size_t s_wgu_l, s_wgu_e; // per layer, expert: [H x 2F], gate/up panels interleaved
  const uint16_t* wd; size_t s_wd_l, s_wd_e;    // per layer, expert: panel-tiled [F x H]
  const uint16_t* wlm;           // panel-tiled [H x V]
  // FP8 (E4M3) feed-forward weights, when ffn_fp8 (then wgu and wd are unused)
  int32_t ffn_fp8;
  const uint8_t* wgu8; size_t s_gu8_l, s_gu8_e; // per layer, expert: gate/up panels interleaved, chunk pairs
  const uint8_t* wd8; size_t s_d8_l, s_d8_e;    // per layer, expert: [F/16][H][16] codes (batches <= 4)
  const uint8_t* wd8p;                           // the same codes in chunk-pair panels [F x H] (larger batches)
  const float* fsc; size_t s_fsc_l, s_fsc_e;    // per layer, expert: [F][4] scales (gate, up, down, 0)
  const float* rope;             // [max_seq][D/2][2] (cos, sin)
  uint16_t* kv; size_t s_kv_l;   // KV pool, layer stride in elements
  // batch (caller-owned)
  int32_t* tokens;
  const int32_t* bt;
  int32_t* seq_lens;
  float* logits;
  int32_t* next_tokens;
  uint32_t flags;
  // scratch
  float* h;      // [B][H] residual stream
  uint16_t* u;   // [2][2][B][H] layer input x = h * gamma_l as the split pair (bf16(x), bf16(x - bf16(x))), buffer l % 2
  float* q;      // [B][QH*D] rotated queries
  float* part;   // [B][KVH][max_splits][G*D + 2G] attention partials (o, m, l)
  uint16_t* o;   // [2][B][QH*D] attention output as the split pair (hi, lo), bf16
  float* ao;     // [KVH][B][H] O projection partials per kv group
  float* ssq;    // [2][B][NB] per column block sums of squares of layer l's input, buffer l % 2
  float* rp;     // [router_ks][B][E] router logit partials
  int32_t* tk_idx; float* tk_w;  // [B][K]
  int32_t* tk_trace;             // optional [L][B][K] record of every layer's routing
  int32_t* route;
  float* gu;     // [B*K][2 K halves][gate, up][F] expert up/gate partial sums
  float* dn;     // [B*K][H] expert outputs
  float* mp;     // fused MoE: [claimer][MK_FUSED_B][H] partial outputs (routing weights applied)
  float* lm_val; int32_t* lm_arg; // [B][n_lm_tasks] LM head argmax candidates
  // synchronisation
  uint32_t* ctr;        // counters of this step
  uint32_t* ctr_clear;  // counters of the next step (cleared by this step), or null
  int32_t n_ctr;
  uint32_t* err;        // device error word
  const mk_task* tasks;
  const int32_t* task_off;   // per workgroup [off[wg], off[wg+1])
  int32_t waits_enabled;     // 0 in kernel-per-op mode (stream order is the dependency)
  uint32_t* trace;           // optional per-task record (8 words): op | layer << 8 | workgroup << 16,
                             // start, waits satisfied, mark 0, mark 1, end, mark 2, mark 3
  int32_t trace_base;        // index of this launch's first task in the trace
  int64_t timeout_ticks;     // wait time limit in s_memrealtime ticks (100 MHz)
  // Tagged hand-offs (batches up to MK_FUSED_B): a producer stores each value
  // with the tag of its step and layer in one 8-byte word, and a consumer
  // polls the words themselves, so no store has to be acknowledged and no
  // counter has to travel before the data is used.
  int32_t tagged;            // 1: the QKV outputs reach attention, and the router's partial
                             // logits the fused MoE claimers, as tagged words
  uint32_t tag_base;         // this step's epoch << 8; layer l's tag is tag_base | (l + 1)
  uint64_t* qt;              // [B][QH*D] rotated queries (float bits | tag << 32)
  uint64_t* kvt;             // [B][KVH][2][D] the new token's key and value (bf16 bits | tag << 32)
  uint64_t* rpt;             // [B*E][4] router logit partials, K split k in word k (float bits | tag << 32)
};

struct mk_handle;
// The shape a decode service needs from a device handle: largest batch, page
// table row stride, pages in the pool, vocabulary. False for a host-only handle.
bool mk_handle_dims(const mk_handle* h, int* max_batch, int* mpps, int* n_pages, int* vocab);
