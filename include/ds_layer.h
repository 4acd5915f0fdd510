/*
 * ds_layer.h -- C ABI of libdslayer.so: one pre-LayerNorm GPT transformer layer with a KV cache,
 * for small-batch decode and for prefill, on one AMD Instinct MI355X (gfx950).
 *
 * What the layer computes follows the customized transformer-block inference kernels described on
 * the page "DeepSpeed Inference 内核优化深度解析：多 GPU 自适应并行、算子融合推理内核与 MoQ 量化支持"
 * (blog.gitcode.com), cited below as [KP]:
 *   [KP] section 三 3.2, region 1: input LayerNorm, then the Q, K, V GeMMs with their bias-adds;
 *   [KP] section 三 3.2, region 2: the head "transform" merged into attention by implicit
 *        addressing (here: K and V rows are written straight into the head-major cache);
 *   [KP] section 三 3.2, region 3: intermediate FF with LayerNorm, bias-add, residual and GELU;
 *   [KP] section 三 3.2, region 4: bias-add and residual on the layer output;
 *   [KP] section 三 3.1: fusion boundaries sit at the two all-reduce points (after the attention
 *        output GeMM and after the layer output GeMM);
 *   [KP] section 五 5.2 and section 四 4.2: int8 weights with group-wise scales (quantize_groups),
 *        dtype fp32 / fp16 / int8 (default fp16), max_out_tokens bounds the generated length.
 * The attention mask follows the triangular_masking option (default true) of the inference-config
 * table on the page "DeepSpeed MoE 大规模稀疏模型推理实战指南" (blog.gitcode.com), cited as [MP].
 *
 * Per new row at absolute position p of sequence b (pre-LN):
 *   h  = LN(x; ln1_g, ln1_b)                  z = W_qkv h + b_qkv = [q | k | v]
 *   K[b][j][p] = k_j, V[b][j][p] = v_j         (head j owns elements [j*d, (j+1)*d))
 *   ctx_j = sum_i softmax_i(q_j . K[b][j][i] / sqrt(d)) V[b][j][i]   over keys i visible to p
 *   x2 = x + W_o ctx + b_o
 *   f  = GeLU(W_ff1 LN(x2; ln2_g, ln2_b) + b_ff1)
 *   y  = x2 + W_ff2 f + b_ff2
 * LayerNorm uses the biased variance; GeLU is u*Phi(u) (erf) or its tanh approximation.
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless marked "host". The caller allocates and owns all device
 *    memory (weights, scales, caches, lengths, activations, workspace); the library only borrows
 *    it. Weights and caches must outlive every call that uses them. A ds_layer_t is a small host
 *    object owned by the library, released by ds_layer_destroy.
 *  - Matrices are [N][K] row-major (K contiguous): W_qkv [3H][H], W_o [H][H], W_ff1 [F][H],
 *    W_ff2 [H][F]. int8 scales are fp16 [N][K/group]: element (n,k) = q[n][k] * s[n][k/group], with
 *    group = quant_group for W_qkv and W_o and the MLP group for W_ff1 and W_ff2.
 *    Every weight, scale, bias, LayerNorm, cache and activation pointer must be 16-byte aligned.
 *  - Enqueueing calls put their work on `stream` (a hipStream_t; NULL is the null stream) and
 *    return without waiting. They allocate nothing and never synchronize, so they can be captured
 *    into a HIP graph.
 *  - Every call returns DS_OK (0) or a negative ds_status. Argument, shape and capacity errors are
 *    found on the host before anything is enqueued and leave all buffers untouched; a failed
 *    launch returns DS_ERR_HIP. ds_last_error() then gives a message (per calling thread).
 *    No C++ exception crosses this interface.
 */
#ifndef DS_LAYER_H
#define DS_LAYER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* DS_BF16: bfloat16 (8-bit significand). A model dtype beside fp16, fp32 and int8 in the config
 * table of "DeepSpeed MoE 大规模稀疏模型推理实战指南" (the dtype row), and the init_inference dtype
 * of "解密DeepSpeed推理引擎：如何让大模型在消费级GPU上跑得更快" section 5.1 (mixed precision: bf16
 * where the device supports it, else fp16). */
typedef enum { DS_F32 = 0, DS_F16 = 1, DS_I8 = 2, DS_BF16 = 3 } ds_dtype;

typedef enum {
  DS_OK = 0,
  DS_ERR_NULL = -1,        /* a required pointer is NULL                                      */
  DS_ERR_SHAPE = -2,       /* inconsistent or unsupported sizes                               */
  DS_ERR_DTYPE = -3,       /* unsupported (weight, activation) dtype pair or group size       */
  DS_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned                                */
  DS_ERR_KV_FULL = -5,     /* the step would write past the cache capacity                    */
  DS_ERR_UNSUPPORTED = -6, /* a valid request this build does not implement                   */
  DS_ERR_HIP = -7,         /* the HIP runtime reported an error                               */
  DS_ERR_WORKSPACE = -8    /* the workspace is smaller than ds_layer_workspace_bytes()        */
} ds_status;

/* The layer description ([KP] section 四 4.2 and section 五 5.2; [MP] config table). */
typedef struct {
  int32_t hidden;             /* H = heads * head_dim; a multiple of 64                         */
  int32_t heads;              /* number of attention heads                                      */
  int32_t head_dim;           /* d: 64 or 128                                                   */
  int32_t ffn;                /* F: intermediate width, a multiple of 64                        */
  int32_t weight_dtype;       /* ds_dtype of W_qkv, W_o, W_ff1, W_ff2                           */
  int32_t act_dtype;          /* ds_dtype of x, y, the caches, biases and LayerNorm parameters  */
                              /* supported pairs: (F32,F32) (F16,F16) (I8,F16) (BF16,BF16)      */
  int32_t quant_group;        /* int8: elements per scale along the reduction dimension of      */
                              /* W_qkv and W_o (and of W_ff1, W_ff2 when quant_group_mlp is 0);  */
                              /* 0 for other weight dtypes                                       */
  int32_t quant_group_mlp;    /* int8: elements per scale of W_ff1 and W_ff2 (0: quant_group)    */
                              /* ([KP] section 五 5.2: quantize_groups and mlp_extra_grouping,   */
                              /* finer groups for the MLP matrices); 0 for other weight dtypes.  */
                              /* Both must be multiples of 16 dividing their matrices' K (hidden */
                              /* for W_qkv, W_o, W_ff1; ffn for W_ff2), else DS_ERR_SHAPE.        */
  float ln_eps;               /* LayerNorm epsilon, > 0 (1e-5 by default)                       */
  int32_t gelu_tanh;          /* 0: u*Phi(u) with erf (default); 1: tanh approximation          */
  int32_t triangular_masking; /* 1 (default): a row at position p sees keys 0..p; 0: all keys   */
  int32_t kv_dtype;           /* 0 (default): the cache holds K and V in act_dtype; DS_I8: int8  */
                              /* codes with one fp16 scale per cached row of one head (k_scale, */
                              /* v_scale of ds_kv_cache), for fp16 or bf16 activations. The     */
                              /* pages do not quantize the cache: this applies their group-wise */
                              /* weight quantizer ([KP] section 五 5.2) with one group per row: */
                              /* scale = fp16_RNE(amax/127), code = clamp(RNE(x/scale), +-127); */
                              /* attention reads q*s, the new rows included.                    */
} ds_layer_desc;

/* Borrowed device pointers to one layer's parameters. s_* are the fp16 group scales of the int8
 * matrices and must be NULL unless weight_dtype is DS_I8. Biases and LayerNorm vectors are in
 * act_dtype. */
typedef struct {
  const void *ln1_g, *ln1_b;
  const void *w_qkv, *b_qkv, *s_qkv;
  const void *w_o, *b_o, *s_o;
  const void *ln2_g, *ln2_b;
  const void *w_ff1, *b_ff1, *s_ff1;
  const void *w_ff2, *b_ff2, *s_ff2;
} ds_layer_weights;

/* A caller-owned KV cache for one layer. k and v are [batch][heads][capacity][head_dim] in
 * act_dtype, or int8 codes when the layer's kv_dtype is DS_I8; k_scale and v_scale are then
 * [batch][heads][capacity] fp16 row scales (NULL otherwise). d_len is a device int32[batch] holding the number of filled rows of each sequence;
 * decode and prefill write the new rows at d_len[b].. and then add the number of new rows to it.
 * h_len is an optional HOST int32[batch] mirror of d_len: when it is not NULL the library checks
 * capacity against it before enqueueing and advances it at enqueue time (a graph replay does not
 * advance it). When h_len is NULL the kernels clamp: a row that would land at or past capacity is
 * not written and the sequence's length is not advanced. */
typedef struct {
  void* k;
  void* v;
  int32_t* d_len;
  int32_t* h_len;
  int32_t batch;
  int32_t capacity;
  void* k_scale;
  void* v_scale;
} ds_kv_cache;

typedef struct ds_layer ds_layer_t;

/* Validates the description and the weight pointers on the host (no device work) and returns a
 * handle that borrows the weights. Errors: DS_ERR_NULL, DS_ERR_SHAPE, DS_ERR_DTYPE, DS_ERR_ALIGN. */
int ds_layer_create(const ds_layer_desc* desc, const ds_layer_weights* weights, ds_layer_t** out);

/* Releases the handle (not the borrowed memory). NULL is accepted. */
int ds_layer_destroy(ds_layer_t* layer);

/* Bytes of device workspace that decode (max_tokens == 1) or prefill needs for up to max_batch
 * sequences of max_tokens new rows against caches of `capacity` rows. For int8 weights and more
 * than 16 rows this includes an fp16 copy of the largest weight matrix (each matrix is expanded
 * there just before its product). Returns 0 on bad input. */
size_t ds_layer_workspace_bytes(const ds_layer_t* layer, int32_t max_batch, int32_t max_tokens,
                                int32_t capacity);

/* Copies ntok new rows of keys and values, k_new and v_new [batch][ntok][hidden] in act_dtype,
 * into cache rows d_len[b] .. d_len[b]+ntok-1 (head j taking elements [j*d,(j+1)*d)), then adds
 * ntok to d_len[b] (and to h_len[b] when given). Used to fill a cache with given past rows. */
int ds_kv_append(const ds_layer_t* layer, ds_kv_cache* kv, const void* k_new, const void* v_new,
                 int32_t batch, int32_t ntok, void* stream);

/* One decode step ([KP] section 三 3.2, regions 1-4) for `batch` sequences of one new row each:
 * x, y [batch][hidden] in act_dtype (y may alias x; no other aliasing). Writes the new K and V
 * rows at d_len[b], attends over rows 0..d_len[b], advances d_len[b] by one. The workspace must
 * hold ds_layer_workspace_bytes(layer, batch, 1, kv->capacity) bytes; its contents need no
 * initialization and are scratch between calls. */
int ds_layer_forward_decode(const ds_layer_t* layer, ds_kv_cache* kv, const void* x, void* y,
                            int32_t batch, void* workspace, size_t workspace_bytes, void* stream);

/* Prefill of `seq` new rows per sequence (the same layer, with the mask of triangular_masking):
 * x, y [batch][seq][hidden] in act_dtype (y may alias x). Fills cache rows d_len[b]..+seq-1 and
 * advances d_len[b] by seq. Workspace: ds_layer_workspace_bytes(layer, batch, seq, capacity). */
int ds_layer_forward_prefill(const ds_layer_t* layer, ds_kv_cache* kv, const void* x, void* y,
                             int32_t batch, int32_t seq, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Group-wise symmetric int8 quantization of float32 weights w [n][k] ([KP] section 五 5.2):
 * per row and per group of `group` consecutive elements along k,
 *   s = fp16_round_nearest_even(amax / 127)   (amax = max |w| over the group, taken in double),
 *   q = clamp(round_half_even(w / s), -127, 127)   (the division in double), q = 0 when s == 0.
 * Writes q int8 [n][k] and s fp16 [n][k/group]. Requires k % group == 0 and group a multiple of 16.
 * Weights must be finite with |w| <= 127 * 65504 (so that every scale is a finite fp16); other
 * inputs give unspecified codes. Enqueued on stream. */
int ds_quantize_i8(const float* w, int8_t* q, void* s, int32_t n, int32_t k, int32_t group,
                   void* stream);

/* Expands int8 weights to float32: w[n][k] = q[n][k] * s[n][k/group], exactly as the GEMV
 * kernels form each weight value. Enqueued on stream. */
int ds_dequantize_i8(const int8_t* q, const void* s, float* w, int32_t n, int32_t k, int32_t group,
                     void* stream);

/* The kernel launches of one layer step, in order, as ds_layer_time_kernels names them. */
typedef enum {
  DS_PART_LN1 = 0,   /* LayerNorm of the input rows (MFMA and skinny paths)                   */
  DS_PART_QKV = 1,   /* region 1: QKV product + bias, k/v into the cache (fp32 path: with LN1) */
  DS_PART_ATTN = 2,  /* region 2: attention over the cache                                    */
  DS_PART_O = 3,     /* output projection + bias + residual                                   */
  DS_PART_LN2 = 4,   /* LayerNorm of x2 (MFMA and skinny paths; advances the lengths)         */
  DS_PART_FF1 = 5,   /* region 3: FF1 + bias + GeLU (fp32 path: with LN2)                      */
  DS_PART_FF2 = 6,   /* region 4: FF2 + bias + residual                                       */
  DS_PART_LEN = 7    /* the length advance (fp32 path)                                        */
} ds_part;

/* Measurement aid, no layer operation (it serves callers that report each kernel's time against
 * its roofline): runs one step of ds_layer_forward_decode (ntok == 1) or ds_layer_forward_prefill
 * (same arguments and effects) with HIP events recorded on `stream` between its kernel launches,
 * after a GPU-side wait of about 200 us so that the host enqueues the whole step before it starts;
 * then waits for the stream and writes each launch's duration ms[i] and its ds_part kinds[i], in
 * launch order. Returns the number of launches (at most max), or a negative ds_status. Not for
 * graph capture (it synchronizes). */
int ds_layer_time_kernels(const ds_layer_t* layer, ds_kv_cache* kv, const void* x, void* y, int32_t batch,
                          int32_t ntok, void* workspace, size_t workspace_bytes, void* stream, float* ms,
                          int32_t* kinds, int32_t max);

/* Measurement aid, no layer operation (no passage of the pages defines it; it serves callers that
 * quote decode bandwidth against what the device reaches, beside the vendor peak): reads the
 * `bytes` bytes of the device buffer `buf` once with 16-byte streaming loads spread over the whole
 * device and XORs a 32-bit digest of the data into the device word *out, so that the reads cannot
 * be elided; the launch time gives the achievable HBM read bandwidth. buf must be 16-byte aligned
 * and bytes a multiple of 16; the caller owns both buffers. Enqueued on stream; DS_ERR_NULL,
 * DS_ERR_ALIGN or DS_ERR_HIP on failure. */
int ds_read_probe(const void* buf, size_t bytes, uint32_t* out, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Persistent multi-layer decode. A stack binds n_layers layers that share one description (same
 * shapes and dtypes) to their caches (caches[l] for layers[l], all of one capacity and at least
 * max_batch sequences) and runs a whole decode step -- regions 1-4 of [KP] section 三 3.2 for every
 * layer in turn -- as one cooperative launch whose workgroups all stay resident; at the phase
 * boundaries of [KP] section 三 3.1 each workgroup waits for exactly the values of the previous
 * phase it reads (stored with tags naming launch, layer and phase). The cache structs are copied:
 * their k, v, d_len and h_len pointers must stay valid for the stack's life.
 * The stack's persistent device state (the layer table, a launch counter, an exit count and an
 * error flag) lives in a caller-owned device buffer of ds_stack_state_bytes(n_layers) bytes,
 * 16-byte aligned, which ds_stack_create initializes (synchronously) and which must stay valid and
 * untouched for the stack's life; the library allocates no device memory.
 * Requirements: 1 <= n_layers <= 511; max_batch 1..4; hidden <= 8192; hidden and ffn multiples of
 * 256 (fp32 weights), 512 (fp16) or 1024 (int8); each cache under 2 GiB. Errors: DS_ERR_NULL,
 * DS_ERR_SHAPE, DS_ERR_ALIGN, DS_ERR_UNSUPPORTED (n_layers above 511 included), DS_ERR_WORKSPACE
 * (state buffer too small), DS_ERR_HIP.
 * ------------------------------------------------------------------------------------------- */
typedef struct ds_stack ds_stack_t;

/* The ends of a generation step (the GPT-Neo-2.7B text-generation example of [KP] section 二):
 * after the last layer, a final LayerNorm and the LM head, logits = W_vocab LN(y; ln_g, ln_b) (no
 * bias), then greedy decoding: the token is the position of the largest logit, the smallest such
 * position on ties. (The example samples; the logits are returned for callers that do.) Borrowed
 * device pointers: ln_g, ln_b [hidden] in act_dtype; w [vocab][hidden] in weight_dtype; s the fp16
 * scales [vocab][hidden/quant_group] when the weights are int8, else NULL. */
typedef struct {
  const void* ln_g;
  const void* ln_b;
  const void* w;
  const void* s;
  int32_t vocab;  /* >= 1; vocab * hidden weight bytes under 2 GiB */
} ds_lm_head;

/* Bytes of the caller-owned state buffer of a stack of n_layers layers (0 if n_layers < 1). */
size_t ds_stack_state_bytes(int32_t n_layers);

/* head: NULL for a stack without the LM head (ds_stack_forward_generate then fails with
 * DS_ERR_UNSUPPORTED), else copied (its pointers must stay valid for the stack's life). */
int ds_stack_create(const ds_layer_t* const* layers, const ds_kv_cache* caches, int32_t n_layers,
                    int32_t max_batch, const ds_lm_head* head, void* state, size_t state_bytes,
                    ds_stack_t** out);
/* Releases the host handle (no device memory is freed; the state buffer is the caller's). */
int ds_stack_destroy(ds_stack_t* stack);

/* Workspace bytes for a step of `batch` sequences (0 if batch is outside 1..max_batch). The
 * workspace holds the tagged values of one launch; the library clears it (with a fill kernel on
 * the call's stream) the first time a stack uses it after another stack did, and again after every
 * 2^19 - 64 launches of one stack, so that no stale value can carry a current tag. Between calls
 * nothing but the stacks may write it. */
size_t ds_stack_workspace_bytes(const ds_stack_t* stack, int32_t batch);

/* Number of workgroups the persistent launch uses (all co-resident on the device). */
int32_t ds_stack_groups(const ds_stack_t* stack);

/* One decode step through all layers: x, y [batch][hidden] in act_dtype (y may alias x). Writes
 * each layer's new K/V row at its d_len[b], attends over rows 0..d_len[b], and after the last
 * layer advances every layer's d_len[b] (and h_len[b] when given) by one. Enqueued on stream.
 * Calls on one stack must not overlap in time (they share its counters). */
int ds_stack_forward_decode(ds_stack_t* stack, const void* x, void* y, int32_t batch,
                            void* workspace, size_t workspace_bytes, void* stream);

/* One whole generation step: ds_stack_forward_decode through every layer (y receives the last
 * layer's output), then the LM head in the same launch. logits: device fp32 [batch][vocab], or NULL
 * to skip storing them; tokens: device int32 [batch], the greedy choice of each sequence. NaN logits
 * give an unspecified token. Same workspace and errors as ds_stack_forward_decode. */
int ds_stack_forward_generate(ds_stack_t* stack, const void* x, void* y, float* logits, int32_t* tokens,
                              int32_t batch, void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code being captured into a HIP graph, tight
 * serving loops, harnesses that forbid allocation): the same step as ds_stack_forward_decode, with
 * the workspace taken from a static device array inside the library (DS_STACK_STATIC_SCRATCH_BYTES,
 * 16 MiB, held on each GPU the library runs on until the process ends) instead of a caller buffer.
 * The call allocates nothing. A step whose workspace (ds_stack_workspace_bytes) exceeds the array
 * returns DS_ERR_WORKSPACE before anything is enqueued. Every call on one GPU shares that GPU's
 * array, which keeps the last call's contents (the library clears it when a different stack used
 * it last): calls that overlap in time on one GPU, from any stacks or streams, race and give
 * undefined results. Same other arguments, outputs and errors as ds_stack_forward_decode. */
#define DS_STACK_STATIC_SCRATCH_BYTES (16u << 20)
int ds_stack_forward_decode_static(ds_stack_t* stack, const void* x, void* y, int32_t batch, void* stream);

/* Synchronizes the device and reports whether a step of this stack hit its wait timeout
 * (DS_ERR_HIP) or not (DS_OK). After a timeout every later launch of the stack leaves at once,
 * before any store, until this call resets the counters; it also copies every layer's device
 * lengths back into the host mirrors (h_len), which were advanced at enqueue time for steps that
 * then did not run, so the stack can run again from the lengths the device holds. */
int ds_stack_check(ds_stack_t* stack);

/* Limit of each wait of the persistent kernel (default 2 s); on expiry the kernel raises an
 * error flag and every workgroup leaves the launch. */
int ds_stack_set_timeout_us(ds_stack_t* stack, int64_t microseconds);

/* ---------------------------------------------------------------- the MoE expert FF
 * The expert feed-forward block of an MoE layer ("DeepSpeed MoE 大规模稀疏模型推理实战指南", the MoE
 * sections: a number of experts per MoE layer, the layer types 'standard' and 'residual'
 * (PR-MoE)). It takes the residual stream after attention, x2, and returns y for T tokens:
 *   h = LN(x2; ln_g, ln_b);  p = softmax over the experts of W_gate h (no bias);
 *   the top_k experts are the k largest p (the smallest index first among equal values);
 *   w_i = p_i / sum of the chosen p (combine 0), or p_i itself (combine 1);
 *   y = x2 + sum_i w_i FF_{e_i}(h)  [+ FF_r(h) for the residual type],
 *   FF(h) = W2 GeLU(W1 h + b1) + b2 (erf GeLU, or tanh with gelu_tanh).
 * The pages name the experts and the types but not the gate: the gate and the combine weights
 * above are this library's reading. The gate decides in fp32 from h rounded to the activation
 * type (the rows the experts see); a near tie may be decided differently in another precision. */
typedef struct {
  int32_t hidden, ffn;        /* H (multiple of 64), F (multiple of 64)                          */
  int32_t experts, top_k;     /* 1..1023 experts; 1..8 chosen per token, top_k <= experts        */
  int32_t weight_dtype;       /* ds_dtype of W1, W2 (experts and residual MLP)                   */
  int32_t act_dtype;          /* ds_dtype of x2, y, W_gate, biases, LN parameters; pairs as for  */
                              /* a layer: (F32,F32) (F16,F16) (I8,F16) (BF16,BF16)               */
  int32_t quant_group;        /* int8: elements per fp16 scale along K of W1 and W2 (a multiple  */
                              /* of 16 dividing hidden and ffn); 0 otherwise                     */
  float ln_eps;               /* > 0                                                             */
  int32_t gelu_tanh;          /* 0: u*Phi(u) with erf; 1: tanh approximation                     */
  int32_t residual;           /* 0: 'standard'; 1: 'residual' (PR-MoE: a dense MLP added)         */
  int32_t combine;            /* 0: chosen p renormalized to sum 1; 1: the softmax p             */
} ds_moe_desc;

/* Borrowed device pointers, all 16-byte aligned. Experts are stacked: W1 [E][F][H], b1 [E][F],
 * W2 [E][H][F], b2 [E][H]; int8 scales s1 [E][F][H/group], s2 [E][H][F/group] (NULL otherwise).
 * W_gate [E][H], ln_g, ln_b [H] are in the activation dtype. r_* are the residual MLP's (one
 * expert's shapes), required for the residual type and NULL for the standard type. */
typedef struct {
  const void *ln_g, *ln_b, *w_gate;
  const void *w1, *b1, *s1, *w2, *b2, *s2;
  const void *r_w1, *r_b1, *r_s1, *r_w2, *r_b2, *r_s2;
} ds_moe_weights;

typedef struct ds_moe ds_moe_t;

/* Validates and keeps the description and pointers (nothing is read from the device). Errors:
 * DS_ERR_NULL, DS_ERR_ALIGN, DS_ERR_SHAPE, DS_ERR_DTYPE. */
int ds_moe_create(const ds_moe_desc* desc, const ds_moe_weights* w, ds_moe_t** out);
int ds_moe_destroy(ds_moe_t* moe);

/* Workspace bytes for steps of up to max_tokens tokens (0 if max_tokens is out of range: tokens
 * times (top_k + residual) may not exceed 4096). */
size_t ds_moe_workspace_bytes(const ds_moe_t* moe, int32_t max_tokens);

/* One step on `tokens` rows of x2 [tokens][H] into y [tokens][H] (y may alias x2). sel_out
 * (int32 [tokens][top_k]) and wgt_out (fp32 [tokens][top_k]) receive the chosen experts and their
 * combine weights when not NULL. Enqueues five kernels on `stream` (gate, routing, the experts'
 * two products, combination); allocates nothing and never synchronizes. Every chosen expert's
 * weights are read once per step, however many tokens chose it. Errors before any enqueue:
 * DS_ERR_NULL, DS_ERR_ALIGN, DS_ERR_SHAPE (tokens < 1 or too many pairs), DS_ERR_WORKSPACE. */
int ds_moe_forward(const ds_moe_t* moe, const void* x2, void* y, int32_t tokens, int32_t* sel_out, float* wgt_out,
                   void* workspace, size_t workspace_bytes, void* stream);

/* The same step with a HIP event after each of the five launches; ms[i] (host, max entries)
 * receives their durations in launch order (0 gate, 1 routing, 2 FF1, 3 FF2, 4 combination).
 * With one slot per token (top_k 1, standard type) FF2 writes y itself and entry 4 is the empty
 * interval after it. Synchronizes the stream. Returns the number of launches or a negative status. */
int ds_moe_time_kernels(const ds_moe_t* moe, const void* x2, void* y, int32_t tokens, void* workspace,
                        size_t workspace_bytes, void* stream, float* ms, int32_t max);

/* Message describing the last non-zero status returned on the calling thread. */
const char* ds_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DS_LAYER_H */
