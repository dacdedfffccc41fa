/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention library.
 *
 * KDA is the gated delta rule with a channel-wise forget gate and one
 * fixed-size state matrix S (d_k x d_v, fp32) per (sequence, head):
 *
 *     S_t = (I - beta_t k_t k_t^T) diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t,           alpha_t = exp(max(g_t, g_floor))
 *
 * Sources (page title, section):
 *   - delta-rule update (erase along k, then write), output read from the
 *     updated state, state of size [d, d_v]: "Kimi K3 深度拆解" (chenxutan.com),
 *     4.2 "线性注意力与 Delta Rule";
 *   - one forget rate per key channel rather than per head: "Kimi K3 技術報告：
 *     三個架構改動一次看懂" (akiraxclaw.com), "長度：KDA 為什麼還要搭配 Gated MLA？";
 *   - fixed-size recurrent state, chunk-parallel computation: "3 分钟看懂
 *     Kimi K3" (landx.limxdynamics.com), "第一条主线";
 *   - lower bound on the log-decay so that every causal chunk, the diagonal
 *     block included, is a dense matrix product: same page, Figure 3; and
 *     "Kimi K3 发布 47 页技术报告" (163.com), section 01;
 *   - decode cost and state size independent of context length: "Kimi K3：
 *     预训练规模与推理算力，必须一起扩展" (studioglobal.ai), "KDA 与 Gated MLA".
 * The pages leave the position of the gate relative to the erase open; this
 * library decays first, as in the formula above.
 *
 * Gate variants (kda_gate_t).  KDA's channel-wise gate extends Gated
 * DeltaNet, where one forget rate per head and token serves every key
 * channel (akiraxclaw.com page above, same section); with no gate at all the
 * recurrence is the plain delta rule (chenxutan.com page above, 4.2).  Both
 * are KDA with alpha_t the same for every channel, or 1:
 *   KDA_GATE_CHANNEL  g is [.., H, d_k]: one log-decay per key channel (KDA);
 *   KDA_GATE_HEAD     g is [.., H]: one log-decay per (token, head), applied
 *                     to every key channel (Gated DeltaNet);
 *   KDA_GATE_NONE     alpha = 1, g is not read and may be NULL (DeltaNet).
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers to contiguous row-major arrays,
 *     16-byte aligned.  The caller owns every buffer; the library allocates
 *     nothing, never synchronises and is reentrant.  Its one piece of global
 *     state is the fixed device scratch of kda_chunk_forward_noalloc.
 *   - Arguments are validated on the host before any launch, so argument
 *     errors come back as status codes even on a machine without a GPU.  The
 *     only HIP calls before the launches are one device-attribute query
 *     (the current device's compute units, which the chunked forward's cut
 *     into segments depends on; 256 when no device answers) and, in
 *     kda_chunk_forward_noalloc, the device address of its scratch.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and is asynchronous: results are valid once the caller synchronises.
 *   - A failed launch returns KDA_ERR_HIP: each launch's own status is
 *     checked (an error that earlier, unrelated HIP calls left on the calling
 *     thread is neither reported nor cleared).  No C++ exception crosses the
 *     ABI.
 *   - Log-decays g must be <= 0 (alpha in (0, 1]); the library applies
 *     max(g, g_floor) itself, which is a no-op on inputs already floored.
 *   - NaN or Inf inputs propagate into the outputs; they never fault or hang.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_VERSION 20000 /* 2.0.0 */

typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARGUMENT = 1, /* NULL pointer, bad size, misalignment, overlap */
  KDA_ERR_UNSUPPORTED = 2,      /* valid but not implemented (e.g. d_k = 96)   */
  KDA_ERR_WORKSPACE_TOO_SMALL = 3,
  KDA_ERR_HIP = 4               /* the HIP runtime reported an error          */
} kda_status_t;

typedef enum { KDA_DTYPE_F32 = 0, KDA_DTYPE_BF16 = 1 } kda_dtype_t;

typedef enum { KDA_GATE_CHANNEL = 0, KDA_GATE_HEAD = 1, KDA_GATE_NONE = 2 } kda_gate_t;

/* Shape of one chunked forward call (the KDA gate: g per key channel). */
typedef struct {
  int B;            /* batch; must be 1 when n_seqs > 0                      */
  int T;            /* tokens per batch row (packed total when n_seqs > 0)   */
  int H;            /* heads                                                 */
  int d_k;          /* key/query channels: 64 or 128 (fp32 chunked: 64)     */
  int d_v;          /* value channels: must equal d_k                        */
  int chunk;        /* tokens per chunk: 64                                  */
  int n_seqs;       /* 0: B sequences of T tokens; > 0: packed sequences     */
  kda_dtype_t dtype;/* dtype of q, k, v, g and o                             */
  float g_floor;    /* per-step log-decay floor, in [-1, 0), |chunk*floor|<=16 */
} kda_chunk_desc_t;

/* The shape and the layout of g, for the entry points that take every gate
 * variant (kda_chunk_forward_gated and the measurement, prefix-cache, MXFP8
 * and backward entry points).  gate = KDA_GATE_CHANNEL is kda_chunk_forward's
 * case exactly. */
typedef struct {
  kda_chunk_desc_t shape;
  kda_gate_t gate;
} kda_chunk_desc_ex_t;

/* Static, human-readable name of a status code; never NULL. */
const char* kda_status_string(int status);

/* KDA_VERSION of the built library. */
int kda_version(void);

/*
 * Bytes of device workspace that kda_chunk_forward (and every forward entry
 * point with the same shape) needs for `d`, on the current device.  No
 * launch; see the conventions above.  Returns KDA_OK or KDA_ERR_* for an
 * invalid or unsupported descriptor.  The workspace holds three d_k x d_v
 * fp32 matrices per (segment, head) when sequences are cut into segments
 * (192 KiB at d = 128; the cut aims at about one workgroup per compute unit
 * over all (segment, head) pairs, so 48 MiB at H = 16 for T = 4,096 as for
 * T = 1,048,576), and 16 bytes per packed sequence.
 */
int kda_chunk_forward_workspace_size(const kda_chunk_desc_t* d, size_t* bytes);

/*
 * Chunked forward ("prefill") over whole sequences.
 *
 * Computes, for every sequence and head, the recurrence above over the
 * sequence's tokens, starting from h0 (or zeros), writing o for every token
 * and the final state to ht.  Internally the sequence is cut into chunks of
 * `chunk` tokens (restarting at every sequence start; the last chunk may be
 * short): the chunk-local work is dense bf16/fp32 matrix products and a
 * triangular solve, then the state is carried from chunk to chunk.  The
 * result equals the token-by-token recurrence up to rounding.
 *
 *   q, k    : [B, T, H, d_k]  dtype
 *   g       : [B, T, H, d_k]  dtype, log-decays (natural log) per key channel
 *   v       : [B, T, H, d_v]  dtype
 *   beta    : [B, T, H]       fp32, write strengths in [0, 1]
 *   h0      : [S, H, d_k, d_v] fp32 or NULL (= zero state); S = n_seqs or B
 *   cu_seqlens: device int32 [n_seqs + 1], cu[0] = 0, non-decreasing,
 *             cu[n_seqs] = T; NULL when n_seqs == 0.  Contents are trusted
 *             (they live on the device); callers validate them beforehand.
 *   o       : [B, T, H, d_v]  dtype, written
 *   ht      : [S, H, d_k, d_v] fp32, written, or NULL; may alias h0 exactly
 *   workspace: device buffer of at least kda_chunk_forward_workspace_size()
 *             bytes, 256-byte aligned; its contents are scratch.
 * o must not overlap any input; ht must not overlap q, k, v, g, beta or o.
 */
int kda_chunk_forward(const kda_chunk_desc_t* d,
                      const void* q, const void* k, const void* v, const void* g,
                      const float* beta, const float* h0,
                      const int32_t* cu_seqlens,
                      void* o, float* ht,
                      void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * kda_chunk_forward for every gate variant: d->gate selects the layout of g,
 *   g : [B, T, H, d_k] (KDA_GATE_CHANNEL), [B, T, H] (KDA_GATE_HEAD) dtype,
 *       or NULL (KDA_GATE_NONE: not read).
 * Workspace: kda_chunk_forward_workspace_size(&d->shape).  Everything else
 * as kda_chunk_forward; with KDA_GATE_CHANNEL the two calls are identical.
 */
int kda_chunk_forward_gated(const kda_chunk_desc_ex_t* d,
                            const void* q, const void* k, const void* v, const void* g,
                            const float* beta, const float* h0,
                            const int32_t* cu_seqlens,
                            void* o, float* ht,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * kda_chunk_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same call with no workspace argument.  Its workspace is a
 * fixed scratch array of KDA_NOALLOC_SCRATCH_BYTES (64 MiB) in the library's
 * device code, one per device, held from the library's load on that device
 * until the process ends; the call itself allocates nothing.  The cut into
 * segments keeps to that size (at H = 16 the best cut needs 48 MiB, and
 * shapes whose best cut needs more take the best one that fits); a call
 * whose smallest cut does not fit (more than about 4 million packed
 * sequences) returns KDA_ERR_WORKSPACE_TOO_SMALL before any launch.  Calls
 * on one device share its scratch: two calls in flight at once on one
 * device (on different streams, or from different threads without ordering)
 * race and give undefined results; calls ordered on one stream are safe.
 * Nothing in the scratch needs clearing between calls.  Everything else as
 * kda_chunk_forward; on the same plan the results are bit-identical to it.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int kda_chunk_forward_noalloc(const kda_chunk_desc_t* d,
                              const void* q, const void* k, const void* v, const void* g,
                              const float* beta, const float* h0,
                              const int32_t* cu_seqlens,
                              void* o, float* ht,
                              void* stream);

/*
 * Measurement twin of kda_chunk_forward_gated: the same call, and in
 * addition hipEventRecord(events[i], stream) before each of the call's
 * launches and events[3] after the last one.  The launches, in stream order:
 *   0: map sweep       (each segment's affine state map, from the inputs)
 *   1: segment scan    (every segment's incoming state)
 *   2: output sweep    (o, the final state, prefix-cache states)
 * so hipEventElapsedTime(events[i], events[i + 1]) is launch i's time.  A
 * launch with nothing to do (no tokens, or one segment per sequence: no maps
 * to build or chain) is skipped, its events still recorded.  events: 4
 * hipEvent_t handles created by the caller (any entry may be NULL: not
 * recorded); the array itself must not be NULL.  No synchronisation.
 * Returns what kda_chunk_forward_gated returns, or KDA_ERR_HIP if recording
 * an event fails.
 */
int kda_chunk_forward_timed(const kda_chunk_desc_ex_t* d,
                            const void* q, const void* k, const void* v, const void* g,
                            const float* beta, const float* h0,
                            const int32_t* cu_seqlens,
                            void* o, float* ht,
                            void* workspace, size_t workspace_bytes,
                            void* stream, void* const* events);

/*
 * kda_chunk_forward_gated with q, k and v in MXFP8 (OCP microscaling): each
 * element is one e4m3 byte (finite-only encoding), and every block of 32
 * consecutive channels of one (token, head) shares a scale byte s meaning
 * 2^(s - 127) (e8m0; 255 is not allowed).  Element value = e4m3(byte) *
 * 2^(s - 127).  The decoded values are exact in bf16, and from there the call
 * is the bf16 path: d->shape.dtype must be KDA_DTYPE_BF16, which is the dtype
 * of g and o.  (K3 trains with MXFP8 activations: "Kimi K3 技術報告：三個架構改動
 * 一次看懂" (akiraxclaw.com), "MoonViT-V2 與低位元訓練也不能省略"; here MXFP8
 * halves the bytes of q, k and v.)
 *   q, k, v             : [B, T, H, d] e4m3 bytes, 16-byte aligned
 *   q/k/v_scale         : [B, T, H, d / 32] scale bytes
 * Everything else as kda_chunk_forward_gated (same workspace size); the scale
 * tensors count as inputs in the overlap rules.
 */
int kda_chunk_forward_mx(const kda_chunk_desc_ex_t* d,
                         const void* q, const uint8_t* q_scale,
                         const void* k, const uint8_t* k_scale,
                         const void* v, const uint8_t* v_scale,
                         const void* g, const float* beta, const float* h0,
                         const int32_t* cu_seqlens,
                         void* o, float* ht,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * States at chunk boundaries, for prefix caching (the system side of a
 * long-context KDA model keeps KDA states and a prefix cache: "3 分钟看懂
 * Kimi K3" (landx.limxdynamics.com), section "第一条主线", the paragraph after
 * Figure 3).
 *
 * kda_chunk_forward_states_count: host only.  *count = the number of state
 * slots kda_chunk_forward_states may write for this descriptor and
 * states_every (>= 1, in chunks): B * floor(T / (states_every * chunk)) for
 * a fixed-length batch, floor(T / (states_every * chunk)) for a packed one
 * (an upper bound there: the lengths live on the device).
 *
 * kda_chunk_forward_states: kda_chunk_forward_gated, and in addition, for
 * every sequence n in order and every m >= 1 with m * states_every * chunk
 * <= len_n, the state after the first m * states_every * chunk tokens of the
 * sequence (what ht would be for that prefix, so a later call can resume
 * from it as h0) is written to
 *   states[slot]  : [H, d_k, d_v] fp32, row-major like ht,
 *   slot = (slots of sequences 0 .. n-1) + m - 1,
 * i.e. states is [count, H, d_k, d_v] with the slots of each sequence
 * consecutive; slots past the last one written are left untouched.
 * states: device buffer of at least count * H * d_k * d_v floats, 16-byte
 * aligned, overlapping no other buffer; it may be NULL only when count is 0.
 * Returns what kda_chunk_forward_gated returns, and KDA_ERR_INVALID_ARGUMENT
 * for states_every < 1 or a states buffer that breaks the rules above.
 */
int kda_chunk_forward_states_count(const kda_chunk_desc_t* d, int states_every, size_t* count);
int kda_chunk_forward_states(const kda_chunk_desc_ex_t* d,
                             const void* q, const void* k, const void* v, const void* g,
                             const float* beta, const float* h0,
                             const int32_t* cu_seqlens,
                             void* o, float* ht,
                             float* states, int states_every,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * Backward pass of kda_chunk_forward_gated (training: K3's KDA layers are
 * trained chunk-parallel up to million-token contexts, "3 分钟看懂 Kimi K3"
 * (landx.limxdynamics.com), "第一条主线"; the pages give no gradient, so it is
 * derived from the recurrence above by the chain rule).
 *
 * Given dout = dL/do and dht = dL/dht for the forward with the same
 * descriptor and inputs, writes the gradients of L with respect to every
 * input:
 *   dq, dk  : [B, T, H, d_k]  dtype          dv: [B, T, H, d_v] dtype
 *   dg      : the layout of g (dtype), or NULL with KDA_GATE_NONE (ignored)
 *   dbeta   : [B, T, H] fp32
 *   dh0     : [S, H, d_k, d_v] fp32, or NULL (not written)
 * dout: [B, T, H, d_v] dtype; dht: [S, H, d_k, d_v] fp32 or NULL (= zero).
 * The floor max(g, g_floor) passes the gradient where g >= g_floor (on the
 * floor itself too: the derivative from above) and gives 0 where g is below.
 * The call replays the forward internally (its outputs are not needed).
 * The workspace (256-byte aligned) holds the replay's state after every
 * chunk (64 KiB per (chunk of 64 tokens, head) at d = 128) and, for the
 * chunks in flight, fp32 records and state gradients (about 0.27 MiB per
 * (chunk, head) at d = 128; at d = 64 also a scratch area).  Chunks are
 * processed in windows of W chunk indices of every sequence, from the last
 * window to the first; the call takes the widest window that fits
 * workspace_bytes (one window for the whole sequence when everything fits),
 * and the results do not depend on it.  kda_chunk_backward_workspace_size gives the default: one
 * window unless the in-flight areas of the whole call would pass 8192
 * (chunk, head) pairs, else windows of max(64, 8192 / (H rows)) chunks.
 * A workspace too small for windows of one chunk is
 * KDA_ERR_WORKSPACE_TOO_SMALL.  Outputs must not overlap each other, the
 * inputs or the workspace.  Other rules as kda_chunk_forward.
 */
int kda_chunk_backward_workspace_size(const kda_chunk_desc_t* d, size_t* bytes);
int kda_chunk_backward(const kda_chunk_desc_ex_t* d,
                       const void* q, const void* k, const void* v, const void* g,
                       const float* beta, const float* h0, const int32_t* cu_seqlens,
                       const void* dout, const float* dht,
                       void* dq, void* dk, void* dv, void* dg, float* dbeta, float* dh0,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_backward with part of its work on a second stream.  Only the
 * local-gradient stage reads what the forward replay writes, so the replay
 * runs beside the state-gradient stage, which fills one CU per (sequence,
 * head, 16 state columns) and leaves the rest idle at small batch.  That stage
 * is then walked in several launches over ranges of the chunks, the last
 * chunks first (four ranges of the chunks, or of each window when the
 * workspace makes windows; two when that span is 64 chunks or fewer), and
 * the local gradients of each range but the
 * first run on the second stream beside the walk over the ranges before it.
 *   aux_stream : hipStream_t (NULL = the default stream) that work is
 *                enqueued on; it waits for `stream` at each fork, and
 *                `stream` waits for it before the call's last launch and
 *                once more at the end.
 *   fork_event, join_event : two distinct caller-created hipEvent_t; both are
 *                re-recorded by every call, so concurrent calls need their own.
 * Results are bit-identical to kda_chunk_backward.  Every work item the call
 * enqueues is ordered before later work on `stream`.  Arguments, workspace
 * and errors as kda_chunk_backward; NULL or equal events are
 * KDA_ERR_INVALID_ARGUMENT.
 */
int kda_chunk_backward_overlapped(const kda_chunk_desc_ex_t* d,
                                  const void* q, const void* k, const void* v, const void* g,
                                  const float* beta, const float* h0, const int32_t* cu_seqlens,
                                  const void* dout, const float* dht,
                                  void* dq, void* dk, void* dv, void* dg, float* dbeta, float* dh0,
                                  void* workspace, size_t workspace_bytes, void* stream,
                                  void* aux_stream, void* fork_event, void* join_event);

/*
 * Measurement twin of kda_chunk_backward: events[i] (5 caller-created
 * hipEvent_t, entries may be NULL) is recorded before stage i and events[4]
 * after the last.  Stages: 0 forward replay (its launches), 1 chunk records,
 * 2 state gradients (reverse over the chunks), 3 local gradients.  With
 * several windows of chunks (a workspace smaller than one window needs),
 * stages 1 to 3 are those of the first window processed (the last chunks)
 * and the interval from events[3] to events[4] also holds the later windows.
 */
int kda_chunk_backward_timed(const kda_chunk_desc_ex_t* d,
                             const void* q, const void* k, const void* v, const void* g,
                             const float* beta, const float* h0, const int32_t* cu_seqlens,
                             const void* dout, const float* dht,
                             void* dq, void* dk, void* dv, void* dg, float* dbeta, float* dh0,
                             void* workspace, size_t workspace_bytes, void* stream,
                             void* const* events);

/*
 * One decode step: one new token for each of N sequences, state resident
 * in device memory and updated IN PLACE.  For every (n, h):
 *     S' = diag(alpha) S;  u = beta (v - S'^T k);  S <- S' + k u^T;
 *     o  = S^T q
 * (the recurrence above for a single token; decode cost and state size do
 * not depend on how many tokens came before).
 *
 *   q, k, g : [N, H, d_k] dtype (g: log-decays per key channel)
 *   v       : [N, H, d_v] dtype
 *   beta    : [N, H] fp32            o: [N, H, d_v] dtype, written
 *   state   : [N, H, d_k, d_v] fp32, read and overwritten
 * d_k = d_v in {64, 128}.  state must not overlap any other argument and o
 * must not overlap any input.
 */
int kda_decode_step(int N, int H, int d_k, int d_v, kda_dtype_t dtype, float g_floor,
                    const void* q, const void* k, const void* v, const void* g,
                    const float* beta, float* state, void* o, void* stream);

/*
 * kda_decode_step for every gate variant: g is [N, H, d_k]
 * (KDA_GATE_CHANNEL), [N, H] (KDA_GATE_HEAD) dtype, or NULL (KDA_GATE_NONE:
 * not read).  With KDA_GATE_CHANNEL identical to kda_decode_step.
 */
int kda_decode_step_gated(int N, int H, int d_k, int d_v, kda_dtype_t dtype, kda_gate_t gate,
                          float g_floor, const void* q, const void* k, const void* v, const void* g,
                          const float* beta, float* state, void* o, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
