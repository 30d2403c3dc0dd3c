/*
 * mk.h - C ABI of the MI355X (gfx950) persistent decode megakernel.
 *
 * One call of mk_decode_step runs one decode step of a parallel-transformer
 * mixture-of-experts decoder for a batch of sequences: embedding, then per
 * layer RMSNorm -> {QKV + RoPE + paged KV append -> split-KV attention ->
 * combine -> O projection} and {router -> top-k -> route finalize -> expert
 * up/gate + SiLU -> expert down -> weighted combine}, rejoined by a fused
 * residual add + RMSNorm; then the final norm, the LM head and the greedy
 * token. Source: Cohere's post on the North Mini Code decode megakernel,
 * sections "What is a Megakernel?" (one persistent workgroup per compute unit
 * walking a host-built task list, global-memory counters for dependencies),
 * "Tasks" (the opcode list), "The task descriptor" and the Chinese version's
 * barrier listing (counters spun on and incremented) and engine section
 * (update page tables, clear barriers, select schedule, launch, sample).
 *
 * Conventions for every entry point:
 *   - Status codes, never exceptions; mk_last_error() gives a message.
 *   - "device" pointers are HIP device memory of the device the handle was
 *     created on; "host" pointers are ordinary host memory.
 *   - bf16 tensors are raw IEEE bfloat16 bit patterns (uint16).
 *   - Streams are hipStream_t passed as void* (NULL = the default stream).
 *   - Argument errors are detected on the host before anything is launched.
 *     Errors found on the device (bad page/token index, a dependency wait
 *     that exceeds its time limit) set a device error word; the kernel then
 *     drains without touching memory further and mk_sync_status() reports it.
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MK_OK = 0,
  MK_ERR_INVALID_ARG = 1,    /* bad pointer, size or shape */
  MK_ERR_UNSUPPORTED = 2,    /* a shape or mode this build does not handle */
  MK_ERR_OOM = 3,            /* device allocation failed */
  MK_ERR_HIP = 4,            /* a HIP runtime call failed */
  MK_ERR_DEVICE_TIMEOUT = 5, /* a dependency wait on the device timed out */
  MK_ERR_DEVICE_FAULT = 6,   /* the device rejected an index (page, token, position) */
  MK_ERR_STATE = 7           /* e.g. decode before all weights were loaded */
} mk_status;

typedef enum { MK_MODE_MEGAKERNEL = 0, MK_MODE_KERNEL_PER_OP = 1 } mk_mode;

/* Model shape and limits.
 * Layer l uses full attention iff window == 0 or l % full_every == full_every-1;
 * other layers attend to the `window` most recent positions including the
 * current one. Query head h reads key/value group h / (n_q_heads / n_kv_heads).
 * RoPE rotates interleaved pairs (2i, 2i+1) by position * theta^(-2i/head_dim).
 * RMSNorm is h / sqrt(mean(h^2) + rms_eps) * gamma. */
typedef struct {
  int32_t hidden;          /* H, a multiple of 256, <= 2048 */
  int32_t n_q_heads;       /* QH */
  int32_t n_kv_heads;      /* KVH <= 8, divides QH; QH / KVH <= 16, (QH / KVH) * D <= 1024 */
  int32_t head_dim;        /* D: 64 or 128 */
  int32_t n_experts;       /* E, a multiple of 8, <= 128 */
  int32_t top_k;           /* k <= 8 */
  int32_t expert_ffn;      /* F, a multiple of 128, <= 768 */
  int32_t vocab;           /* V, a multiple of 16 */
  int32_t n_layers;        /* L */
  float rope_theta;
  float rms_eps;
  int32_t page_size;       /* tokens per KV page: 16 */
  int32_t window;          /* 0 = all layers full attention */
  int32_t full_every;      /* >= 1 */
  int32_t max_batch;       /* largest batch mk_decode_step will be called with, <= 32 */
  int32_t max_seq_len;     /* largest seq_len (positions + 1) any step may see */
  int32_t max_pages_per_seq; /* row stride of block_tables */
  int32_t n_pages;         /* pages in the KV pool */
  int32_t mode;            /* mk_mode */
  int32_t dense;           /* 0: parallel MoE layers (above). 1: dense sequential
                            * layers, h += Attn(RMSNorm(h; gamma)), then
                            * h += FFN(RMSNorm(h; gamma2)) with one SwiGLU FFN of
                            * width expert_ffn (a multiple of 128, <= 8192);
                            * n_experts = top_k = 1, no router, max_batch <= 4
                            * (the Llama-3.2-1B decode path of the tiny-vllm
                            * walkthrough, section "The remaining layers and
                            * logits"; the post's FFN_UPGATE_ACT and FFN_DOWN,
                            * section "Tasks") */
  int32_t ffn_fp8;         /* 0: bf16 feed-forward weights. 1: FP8 (OCP E4M3)
                            * feed-forward weights, one float32 scale per hidden
                            * unit for each of its gate column, up column and
                            * down row, loaded with mk_load_ffn_fp8; the other
                            * weights stay bf16; above 4 sequences the MoE is
                            * the claiming variant at every batch. (The post's
                            * roadmap: FP8 weights, Chinese version, section
                            * "下一步".) */
} mk_config;

typedef struct mk_handle mk_handle;

/* Create a decoder for `cfg` on HIP device `device` (the handle the engine
 * around the kernel drives step by step: megakernel post, Chinese version,
 * section "内核周围的推理引擎", the C++ decode service).
 * kv_pool: the paged KV cache, bf16, in the layout
 *   [n_layers][n_pages][2][n_kv_heads][page_size * head_dim]
 *   plane 0 = K, element (slot s, dim d) at s*head_dim + d;
 *   plane 1 = V, stored transposed: element (slot s, dim d) at d*page_size + s.
 * Page p of a sequence holds its positions [p*page_size, (p+1)*page_size)
 * (tiny-vllm decode walkthrough, section on scattering K/V into blocks).
 * Either the caller owns it (kv_pool = device pointer, 16-byte aligned,
 * valid until mk_destroy, kv_pool_bytes = the size of that layout), or
 * kv_pool = NULL and kv_pool_bytes = 0: the library allocates it, zeroed,
 * frees it in mk_destroy, and mk_kv_cache gives its address.
 * Allocates the library's weight copy (uninitialised), scratch and counters.
 * Errors: MK_ERR_INVALID_ARG / MK_ERR_UNSUPPORTED for the config or the
 * pool, MK_ERR_OOM, MK_ERR_HIP; nothing is left allocated on failure. */
mk_status mk_create(const mk_config* cfg, void* kv_pool, size_t kv_pool_bytes,
                    int device, mk_handle** out);

/* Layer `layer`'s part of the KV pool: *kv_base (device) and *bytes, in the
 * layout above. Valid until mk_destroy; the caller may write context K/V
 * there (synthetic context, or a prefill's output: the post's engine section
 * has ordinary prefill kernels fill the pages while the decode service is
 * parked) when no step is in flight. */
mk_status mk_kv_cache(mk_handle* h, int layer, void** kv_base, size_t* bytes);

/* Load one layer's weights from caller-owned device bf16 tensors in the
 * canonical row-major [in x out] layout; the library repacks them into its own
 * copy (so the caller may free them once `stream` has passed this call). The
 * tensors are the parallel layer's (megakernel post, section "减少波量化":
 * attention and the MoE read one normalised input; section "任务": QKV and O
 * projections, router, expert gate/up and down). Errors: MK_ERR_INVALID_ARG
 * (layer, null or misaligned pointer), MK_ERR_HIP.
 *   gamma [H]; wqkv [H][QH*D + 2*KVH*D] (q heads, then k heads, then v heads);
 *   wo [QH*D][H]; wr [H][E]; wg, wu [E][H][F]; wd [E][F][H].
 * A dense model's layers load through mk_load_layer_dense (MK_ERR_INVALID_ARG
 * here). */
mk_status mk_load_layer(mk_handle* h, int layer, const void* gamma, const void* wqkv,
                        const void* wo, const void* wr, const void* wg, const void* wu,
                        const void* wd, void* stream);

/* One dense sequential layer's weights (cfg.dense = 1; the tiny-vllm
 * walkthrough's layer: attention norm, QKV, O projection, post-attention
 * norm, gate, up, down), caller-owned device bf16 tensors in the canonical
 * row-major [in x out] layout, repacked like mk_load_layer's:
 *   gamma [H]; wqkv [H][QH*D + 2*KVH*D]; wo [QH*D][H]; gamma2 [H];
 *   wg, wu [H][F]; wd [F][H].
 * Errors: MK_ERR_INVALID_ARG (not a dense model, layer, null or misaligned
 * pointer), MK_ERR_HIP. */
mk_status mk_load_layer_dense(mk_handle* h, int layer, const void* gamma, const void* wqkv,
                              const void* wo, const void* gamma2, const void* wg, const void* wu,
                              const void* wd, void* stream);

/* One layer's FP8 feed-forward weights (cfg.ffn_fp8 = 1; the post's roadmap
 * of narrower weight types, Chinese version, section "下一步"): caller-owned
 * device tensors, repacked into the library's copy (free them once `stream`
 * has passed this call):
 *   wg8, wu8 [E][H][F] and wd8 [E][F][H]: OCP FP8 E4M3 codes (uint8), the
 *   canonical row-major layouts of mk_load_layer (a dense model: E = 1);
 *   sg, su, sd [E][F] float32: hidden unit f's gate column is
 *   e4m3(wg8[e][:, f]) * sg[e][f], its up column likewise with su, its down
 *   row e4m3(wd8[e][f][:]) * sd[e][f].
 * Codes 0x7F and 0xFF (NaN) are not valid weights. An FP8 model's
 * mk_load_layer / mk_load_layer_dense / mk_load_weights calls pass NULL for
 * wg, wu and wd; a step needs both calls made for every layer.
 * Errors: MK_ERR_INVALID_ARG (not an FP8 model, layer, null or misaligned
 * pointer), MK_ERR_STATE (host-only handle), MK_ERR_HIP. */
mk_status mk_load_ffn_fp8(mk_handle* h, int layer, const void* wg8, const void* wu8, const void* wd8,
                          const float* sg, const float* su, const float* sd, void* stream);

/* Load the embedding [V][H], final norm gain [H] and LM head [H][V] (bf16),
 * caller-owned device tensors, copied or repacked like mk_load_layer's
 * (section "任务": LM_HEAD). A model whose head is tied to the embedding
 * passes the embedding's transpose as wlm. */
mk_status mk_load_globals(mk_handle* h, const void* emb, const void* gamma_f,
                          const void* wlm, void* stream);

/* All weights at once: arrays of n_layers device pointers per tensor kind
 * (host arrays of device pointers); the same checks as the calls above. A
 * dense model gives gamma2 and leaves wr NULL; a MoE model leaves gamma2
 * NULL. An FP8 model (cfg.ffn_fp8) leaves wg, wu and wd NULL and loads its
 * feed-forward weights with mk_load_ffn_fp8. */
typedef struct {
  const void* emb;
  const void* gamma_f;
  const void* wlm;
  const void* const* gamma;
  const void* const* wqkv;
  const void* const* wo;
  const void* const* wr;
  const void* const* wg;
  const void* const* wu;
  const void* const* wd;
  const void* const* gamma2; /* dense models: the FFN's norm gains */
} mk_weights;
mk_status mk_load_weights(mk_handle* h, const mk_weights* w, void* stream);

/* Flags of mk_decode_step. */
#define MK_STEP_ADVANCE 1u /* after the step: tokens[b] = next token, seq_lens[b] += 1 */

/* One decode step for `batch` sequences, enqueued on `stream` (no host sync):
 * one launch of the persistent kernel over the schedule prebuilt for
 * (batch, context bucket) (megakernel post, section "什么是 Megakernel？";
 * engine section: select_schedule(max_live_context()), launch; barriers are
 * cleared by the previous step's kernel, section "屏障").
 *   tokens       device int32 [batch]: token being decoded per sequence
 *   block_tables device int32 [batch][max_pages_per_seq]: physical page ids;
 *                entries for pages holding positions < seq_len must be valid
 *   seq_lens     device int32 [batch]: length INCLUDING this token; the token
 *                sits at position seq_len - 1, and its K/V are appended there
 *                before attention reads the cache
 *   max_seq_len_hint host: an upper bound of seq_lens in this step (selects
 *                the cached schedule; the device clamps nothing to it, it
 *                rejects lengths beyond it with MK_ERR_DEVICE_FAULT)
 *   logits       device float32 [batch][vocab], written
 *   next_tokens  device int32 [batch] or NULL: greedy token (argmax, lowest
 *                index on ties)
 * The caller owns every argument buffer and keeps it unchanged until the
 * stream has passed the step. Consecutive steps on one handle must be on the
 * same stream or otherwise ordered (they share scratch and counters). */
mk_status mk_decode_step(mk_handle* h, int batch, int32_t* tokens, const int32_t* block_tables,
                         int32_t* seq_lens, int max_seq_len_hint, float* logits,
                         int32_t* next_tokens, uint32_t flags, void* stream);

/* mk_decode_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, semantics and kernels; the step's scratch (activations,
 * partial results, routing, counters, error word) lives in a static device
 * array of MK_STATIC_SCRATCH_BYTES (64 MiB) that each device the library runs
 * on holds until the process ends, instead of the handle's buffers. It calls
 * no allocating routine: a fill kernel zeroes the counters, then the step
 * launches.
 *   - The schedule for (batch, context bucket of max_seq_len_hint) must
 *     already be cached on the handle (built by an earlier mk_decode_step or
 *     mk_schedule_info_get with those sizes): otherwise MK_ERR_STATE.
 *   - A model and max_batch whose step scratch exceeds the array:
 *     MK_ERR_UNSUPPORTED (the full-size model fits up to batch 32 at 16K).
 *   - Every call on one device shares that device's array and keeps the last
 *     call's contents: calls that overlap on one device (other streams, other
 *     handles, other threads) race and must be serialised by the caller.
 *   - mk_sync_status reports device errors of these steps too. */
mk_status mk_decode_step_noalloc(mk_handle* h, int batch, int32_t* tokens, const int32_t* block_tables,
                                 int32_t* seq_lens, int max_seq_len_hint, float* logits,
                                 int32_t* next_tokens, uint32_t flags, void* stream);

/* Switch between the persistent megakernel and the kernel-per-op variant
 * (the same op bodies launched once per wave of same-type tasks, with the
 * stream order in place of the counter waits: the separate-kernels baseline
 * of the post's section "加速从何而来"). Takes effect at the next step;
 * steps must not be in flight on another stream. */
mk_status mk_set_mode(mk_handle* h, int mode);

/* Record, for every task of later steps, eight uint32 into `trace` (device,
 * n_records * 8 words): {opcode | layer << 8 | workgroup << 16, start,
 * dependencies satisfied, inputs loaded, computed, end, 0, 0}, times on the
 * 100 MHz device clock (low 32 bits; 0 where an op records no mark). Megakernel records are indexed like the exported schedule (CU-major),
 * kernel-per-op records in the flattened task order. NULL stops recording;
 * a step whose schedule has more tasks than n_records fails with
 * MK_ERR_INVALID_ARG. */
mk_status mk_set_task_trace(mk_handle* h, uint32_t* trace, size_t n_records);

/* Record every layer's routing of later steps into `trace` (device int32
 * [n_layers][batch][top_k], expert ids in descending router-logit order, ties
 * to the lower id); NULL stops recording. For checking routing decisions. */
mk_status mk_set_routing_trace(mk_handle* h, int32_t* trace);

/* Schedule knobs (megakernel post, Chinese version, section "任务调度器：将任务映射到
 * SM": the host builds named waves per layer, picks their order, flattens them
 * and places task k on unit k mod n; an ablation there compares wave orders
 * and a dependency-affinity placement).
 *   wave order: MK_ORDER_SHIPPED   router, qkv, attention, MoE, O-proj, residual
 *               MK_ORDER_QKV_FIRST qkv before router, otherwise shipped
 *               MK_ORDER_ATTENTION_FIRST  O-proj before the MoE claimers
 *   placement:  MK_PLACE_TUNED       round-robin, except MoE claimers on units
 *                                    without attention work, O projections on
 *                                    the attention units, residual tasks on
 *                                    units free of the next layer's first tasks
 *               MK_PLACE_ROUND_ROBIN task k on unit k mod n, nothing else
 *               MK_PLACE_AFFINITY    tuned, but each attention claimer on the
 *                                    unit of a QKV task it waits for and each
 *                                    residual task on the unit of its column
 *                                    block's first O projection
 *               MK_PLACE_COST_MODEL  the claimers as tuned; every other task,
 *                                    in list order, on the unit where a cost
 *                                    model (bytes streamed per unit, a hop per
 *                                    dependency) says it finishes first (the
 *                                    greedy scheduler of the post's section on
 *                                    the other schedulers it tried)
 *               MK_PLACE_RANDOM      every wave over a random permutation of
 *                                    the units, seeded by mk_set_placement_seed
 *                                    (one candidate of that section's
 *                                    brute-force search)
 * Every combination decodes the same step (only timing and, in the fused MoE
 * of at most 4 tokens, the grouping of the claimers' partial sums change).
 * Drops the cached schedules (synchronises the device); no step may be in
 * flight on another stream. MK_ERR_INVALID_ARG for an unknown value. */
enum { MK_ORDER_SHIPPED = 0, MK_ORDER_QKV_FIRST = 1, MK_ORDER_ATTENTION_FIRST = 2 };
enum { MK_PLACE_TUNED = 0, MK_PLACE_ROUND_ROBIN = 1, MK_PLACE_AFFINITY = 2, MK_PLACE_COST_MODEL = 3,
       MK_PLACE_RANDOM = 4 };
mk_status mk_set_schedule_options(mk_handle* h, int wave_order, int placement);

/* The seed of MK_PLACE_RANDOM's candidate (default 1). Drops the cached
 * schedules like mk_set_schedule_options. */
mk_status mk_set_placement_seed(mk_handle* h, uint64_t seed);

/* Debug: with on != 0, fill every per-step scratch buffer before each step
 * (activations, partials, routing, LM-head candidates; not the KV pool, the
 * counters or the error word) with NaN (float 0xffffffff, bf16 0xffff), the
 * index buffers with 0 and tagged words with NaN and tag 0, so that a task
 * reading a value before its producer wrote it turns the logits to NaN or
 * the step into a device fault report instead of passing with stale data
 * (the post's barrier section warns that a wrong arrival count can let
 * readers drift and fail much later). A correct schedule decodes the same
 * step bit for bit either way. Extra fill kernels on the step's stream. */
mk_status mk_set_debug_poison(mk_handle* h, int on);

/* Time limit of one dependency wait on the device, in microseconds (0: the
 * default, 2 s). A wait that exceeds it sets the device error word
 * (MK_ERR_DEVICE_TIMEOUT) and every workgroup drains to the end of its task
 * list (the post warns that a wrong arrival count deadlocks: section "屏障").
 * Takes effect at the next step. At batches up to 4 the queries and the new
 * key and value reach attention as tagged words (each 8-byte word holds the
 * value and a tag naming the step and layer, polled by the reader instead of
 * a counter); a poll that exceeds the limit reports the same error, with
 * 0xffff0000 | word index in place of the counter index. */
mk_status mk_set_wait_limit(mk_handle* h, uint32_t microseconds);

/* Synchronise `stream` and report any device-side error of earlier steps
 * (MK_ERR_DEVICE_TIMEOUT / MK_ERR_DEVICE_FAULT); clears the error word and the
 * step counters, so the next step starts clean. */
mk_status mk_sync_status(mk_handle* h, void* stream);

/* Diagnostic: read `bytes` of device memory at `buf` once, in 16-byte
 * nontemporal loads spread over every compute unit, on `stream` (async). The
 * time it takes is the practical streaming-read ceiling that the decode
 * step's achieved bandwidth is set against (the pages' speed-of-light
 * argument assumes the weights stream at the HBM rate: megakernel post,
 * introduction); reading a buffer larger than the last-level cache also
 * evicts it, so a timed step after it reads from HBM. `buf` must be 16-byte
 * aligned and `bytes` a nonzero multiple of 16 (else MK_ERR_INVALID_ARG,
 * message through mk_last_error(NULL)); nothing is written. */
mk_status mk_stream_read(const void* buf, size_t bytes, void* stream);

/* Diagnostic: the cross-XCD message-passing litmus of the protocol every
 * hand-off between compute units uses (device-coherent stores, a drain, then
 * a relaxed device-scope atomic on a counter; the reader polls the counter and
 * reads device-coherently; the post's barrier section relies on the same
 * release/acquire order with fences). `pairs` producer/consumer workgroup
 * pairs on different XCDs pass `rounds` 16-word messages each on device
 * `device` (synchronous; allocates and frees its own buffers). *stale: words
 * a consumer read older than the round it had been signalled for; *timeouts:
 * waits that gave up (20 ms each; a pair stops at its first timeout or stale
 * read, so the kernel always ends). coherent = 0 uses plain loads and stores
 * for the message instead (the contrast). coherent = 2 checks the tagged
 * hand-off instead: the producer stores 16 words of (value, round) with one
 * 8-byte device-coherent store each and neither drains nor signals; the
 * consumer polls the words (16-byte loads) until every tag is the round's,
 * and *stale counts words whose value is not the one stored with that tag.
 * MK_ERR_INVALID_ARG for pairs outside [1, 512], rounds outside [1, 1e6],
 * coherent outside [0, 2] or null outputs. */
mk_status mk_litmus_message_passing(int device, int pairs, int rounds, int coherent, uint32_t* stale,
                                    uint32_t* timeouts);

/* Last error message of this handle (or of the last failed mk_create when h is NULL). */
const char* mk_last_error(const mk_handle* h);

void mk_destroy(mk_handle* h);

/* Copy `bytes` of one of the library's per-step scratch buffers to host
 * memory after synchronising the device (for op-level checks of the last
 * step's last layer). Names and float32/int32 layouts:
 *   "h" [max_batch][H] residual stream (after the step: the final layer's)
 *   "ssq" [max_batch][H/CB] its per column block sums of squares
 *   "q" [max_batch][QH*D] rotated query   "o" [max_batch][QH*D] attention out
 *   "ao" [KVH][max_batch][H] O-proj partial per kv group
 *   "rp" [K splits][max_batch][E] router logit partial sums
 *   "tk_idx"/"tk_w" [max_batch][k]        "route" expert work queue
 *   "gu" [max_batch*k][2][2][F] expert gate/up sums per K half
 *   "dn" [max_batch*k][H] expert outputs (slot b*k + j). */
mk_status mk_debug_read(mk_handle* h, const char* name, void* host, size_t bytes);

/* ---- schedule introspection (host only, no device work) ---------------- */

/* Task counts of the schedule for (batch, max_seq_len_hint) (section
 * "任务调度器：将任务映射到 SM": per-SM task lists built on the host): total tasks and
 * the longest per-CU list, and the number of dependency counters. */
typedef struct {
  int32_t n_tasks;
  int32_t max_tasks_per_cu;   /* longest task list of one resident workgroup */
  int32_t n_counters;
  int32_t n_cus;              /* resident workgroups (task lists): one per compute unit */
  int64_t weight_bytes_per_step; /* weights streamed at batch 1 routing (k experts) */
} mk_schedule_info;
mk_status mk_schedule_info_get(mk_handle* h, int batch, int max_seq_len_hint, mk_schedule_info* out);

/* Copy the schedule's descriptors (n_tasks * 32 int32, list-major, each
 * resident workgroup's list in execution order) and per-list offsets
 * (n_cus + 1 int32) to host buffers sized from mk_schedule_info_get. */
mk_status mk_schedule_export(mk_handle* h, int batch, int max_seq_len_hint, int32_t* tasks,
                             int32_t* cu_offsets);

/* Run the schedule on a host model of the device (the post's advice to check
 * a schedule's barrier counts before running it: section "你如何编写一个
 * megakernel？"): each CU executes its list
 * in order, a task runs once its counter waits are met, claimers drain their
 * queues; n_active_experts[l] gives the routing outcome per layer (number of
 * distinct experts). Reports deadlock (a state where no CU can progress) and
 * checks every counter's final value against the arrivals it expects.
 * `interleave_seed` picks the order in which ready CUs advance.
 * Returns MK_OK if the run completes and every check holds. */
mk_status mk_schedule_simulate(mk_handle* h, int batch, int max_seq_len_hint,
                               const int32_t* n_active_experts, uint64_t interleave_seed,
                               int32_t corrupt_task, char* report, size_t report_len);

/* Check the schedule for read-before-arrive and overwrite-before-read
 * hazards (the post's barrier section: a wrong arrival count lets a task read
 * before its producer finished): every buffer a task reads or writes is tagged
 * with the writers of its current version and the readers since, in list
 * order; a read must be preceded, through the counters the task waited for
 * (or its unit's earlier tasks), by every writer of the version it reads, and
 * a write by every reader and writer of the version it replaces. Reads are
 * placed where the device code issues them (before, between or after the
 * waits). Accesses among the claimers of one wave, which synchronise through
 * their own item counters, are not modelled. `flags`: 0, or
 * MK_CHECK_EARLY_STREAM_READ to model an earlier device version whose residual
 * task read the residual stream before its waits. MK_OK when no hazard is
 * found, MK_ERR_STATE with the first few in `report` otherwise.
 * MK_CHECK_PLANT_MISSING_WAIT checks a schedule whose residual tasks skip
 * their wait for their contributions (a planted mistake the check must
 * report). */
#define MK_CHECK_EARLY_STREAM_READ 1u
#define MK_CHECK_PLANT_MISSING_WAIT 2u
mk_status mk_schedule_check(mk_handle* h, int batch, int max_seq_len_hint, uint32_t flags, char* report,
                            size_t report_len);

/* Create a handle without any device (schedule introspection and simulation
 * only; mk_load_*, mk_decode_step return MK_ERR_STATE). */
mk_status mk_create_host_only(const mk_config* cfg, int n_cus, mk_handle** out);

/* ---- decode service (megakernel post, Chinese version, section on the
 * inference engine around the kernel: a native thread only decodes, step
 * after step - update the page tables, select the schedule for the longest
 * live context, launch, sample and stream, retire finished requests - while
 * a control-plane thread pauses it to prefill, admit or evict and resumes
 * it; the batch state belongs to the control plane only while the decoder is
 * parked) ------------------------------------------------------------------ */

/* Called from the service thread for every token: status 0 more follow, 1
 * the request finished (max_new_tokens reached or the stop token), -1 the
 * service failed (token is -1; see mk_service_last_error). It runs while the
 * service holds its lock: it must not call mk_service_* functions. */
typedef void (*mk_token_fn)(void* user, int64_t request_id, int32_t token, int32_t status);

typedef struct {
  int32_t max_batch;   /* sequences decoded together, <= the handle's max_batch */
  int32_t page0;       /* the service owns KV pages [page0, page0 + n_pages) of the pool */
  int32_t n_pages;
  mk_token_fn on_token;
  void* user;
  void* stream;        /* hipStream_t of the steps; NULL: a stream of the service's own */
} mk_service_config;

typedef struct {
  int64_t steps;       /* decode steps run */
  int64_t tokens;      /* tokens streamed */
  int32_t active;      /* requests in the batch */
  int32_t free_pages;  /* pages in the service's free list */
  int32_t parked;      /* 1 while the decoder is parked */
  int32_t status;      /* MK_OK, or the error that stopped the service */
} mk_service_info;

typedef struct mk_service mk_service;

/* Start a service thread over handle h (loaded weights, a KV pool; the
 * handle must outlive the service and no one else may step it meanwhile).
 * It starts paused (parked): admit requests, then mk_service_resume. Errors: MK_ERR_INVALID_ARG (config against the
 * handle), MK_ERR_STATE (host-only handle), MK_ERR_OOM. */
mk_status mk_service_create(mk_handle* h, const mk_service_config* cfg, mk_service** out);

/* Ask the decoder to park after its current step and wait until it has: the
 * GPU is idle and the service reads no batch state until mk_service_resume. */
mk_status mk_service_pause(mk_service* s);
mk_status mk_service_resume(mk_service* s);

/* While paused: take n pages from the service's free list (for a request's
 * context, written into the pool through mk_kv_cache, e.g. by a prefill). */
mk_status mk_service_alloc_pages(mk_service* s, int32_t n, int32_t* pages);

/* While paused: admit a request whose context (positions < context_len) is in
 * the KV pool on `pages` (page i holds positions [16 i, 16 i + 16), at least
 * ceil(context_len / 16) of them, from mk_service_alloc_pages). It decodes
 * first_token at position context_len, then greedily, streaming every token
 * through on_token until max_new_tokens or stop_token (-1: none). The
 * service owns the pages from now on and returns them to its free list when
 * the request finishes or is evicted. MK_ERR_UNSUPPORTED when the batch is
 * full, MK_ERR_STATE when not paused. */
mk_status mk_service_admit(mk_service* s, int64_t request_id, int32_t first_token, int32_t context_len,
                           const int32_t* pages, int32_t n_pages, int32_t max_new_tokens, int32_t stop_token);

/* While paused: drop a request (no more tokens; its pages return). */
mk_status mk_service_evict(mk_service* s, int64_t request_id);

mk_status mk_service_stats(mk_service* s, mk_service_info* out);
const char* mk_service_last_error(const mk_service* s);

/* Stop the thread after its current step and free the service (requests
 * still active get no further tokens). */
void mk_service_destroy(mk_service* s);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
