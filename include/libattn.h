/*
 * libattn.h -- C ABI of libattn, multi-head scaled-dot-product self-attention
 * (forward and backward) for AMD Instinct MI355X (gfx950).
 *
 * What is computed.  For a GPT-2 style packed input qkv of shape (B, T, 3C)
 * split into NH heads of size hs = C/NH, every head (b, h) and query row t
 * attends to the key set U(t) = {0..t} (causal) or {0..T-1} (non-causal):
 *
 *     s[t,j]   = q_t . k_j                              (unscaled dot product)
 *     att[t,j] = exp(scale*s[t,j]) / sum_{j' in U(t)} exp(scale*s[t,j'])
 *     out_t    = sum_{j in U(t)} att[t,j] v_j,         scale = 1/sqrt(hs)
 *
 * This is Scores = Q K^T / sqrt(d_k), a softmax per row and a product with V
 * ("Umakini wa kujitegemea, kerneli za CUDA na FlashAttention", section 1),
 * with the causal row set, the packed layout and the unscaled preatt of the
 * CPU references attention_forward_cpu / attention_backward_cpu in llm.c
 * dev/cuda/attention_backward.cu.  The fused entry points never form the
 * T x T matrices: they tile Q, K, V through on-chip memory with a running
 * (online) softmax and keep only a per-row log-sum-exp, which the backward
 * uses to recompute the probabilities (the FlashAttention part of the same
 * page).  The backward is the analytic one of attention_backward_cpu, with
 * the closed-form softmax gradient of softmax_autoregressive_backward_kernel7
 * in attention_backward.cu:
 *
 *     dpreatt[t,j] = scale * att[t,j] * (datt[t,j] - D[t]),
 *     D[t] = sum_j att[t,j] datt[t,j] = dout_t . out_t,  datt[t,j] = dout_t . v_j
 *     dq_t = sum_j dpreatt[t,j] k_j,  dk_j = sum_t dpreatt[t,j] q_t,
 *     dv_j = sum_t att[t,j] dout_t.
 *
 * Layouts (all row-major, contiguous, element strides implied by the shape):
 *     qkv, dqkv   (B, T, 3C): q at [b,t,h*hs+i], k at [b,t,C+h*hs+i],
 *                             v at [b,t,2C+h*hs+i]
 *     out, dout   (B, T, C) : [b,t,h*hs+i]
 *     lse         (B, NH, T): float, natural log, scaled domain:
 *                             lse = log sum_{j in U(t)} exp(scale*s[t,j])
 *     preatt, att, datt, dpreatt (B, NH, T, T): float
 *
 * Pointers.  Every tensor pointer is a DEVICE pointer on the current HIP
 * device, 16-byte aligned, owned by the caller; libattn never frees it.
 * bf16 tensors are passed as uint16_t bit patterns (bfloat16, round to
 * nearest even on output).  Outputs are overwritten (=), never accumulated,
 * except the dq third of dqkv in attn_backward_dkdvdq, which that stage adds
 * to.  An output may not overlap any input or another output.
 *
 * Streams.  Calls enqueue work on the calling thread's libattn stream
 * (attn_set_stream; default: the null stream) and return without waiting.
 * Results are deterministic (fixed reduction order), with one exception: the
 * dq third of the fp32 attn_backward, attn_backward_noalloc and
 * attn_backward_dkdvdq is summed with float atomics, so its last bits may
 * differ from run to run (dk, dv and everything else are bitwise
 * reproducible; the stages attn_backward_dq + attn_backward_dkdv give a
 * reproducible fp32 dq).
 *
 * Workspace.  attn_backward, attn_backward_bf16 and attn_backward_f16 need
 * B*NH*T floats of scratch for D (the 16-bit ones not for the shapes they
 * run as one kernel, see attn_backward_bf16), attn_decode* room for their partial
 * results (4*B*NH*(hs+1)*ceil(T/128) bytes at most), layernorm_backward*
 * room for column partial sums.  libattn keeps one grow-only buffer per
 * device, allocated with hipMalloc on first need.  A call that needs more
 * allocates a larger buffer and retires the old one without freeing it, so
 * growing never synchronises the device and never frees memory that queued
 * work or a captured HIP graph still uses; attn_release() frees the current
 * and every retired buffer.  Calls that use the workspace share it, so such
 * calls on one device must not overlap in time (calls on one stream never
 * do).  HIP graphs: a captured call keeps the workspace address it saw, and
 * a call that grows the workspace allocates, which stream capture may
 * forbid; capture only after an eager call of the same or a larger shape
 * has sized the workspace, or capture the stage calls, which take
 * caller-owned buffers and allocate nothing.  With the environment variable
 * ATTN_TEST_FAIL_ALLOC=1 that allocation fails (ATTN_EHIP) before any HIP
 * call, so callers can test their error handling on any host.
 *
 * Errors.  Every int-returning call returns ATTN_OK or a negative status and
 * records a message for attn_last_error().  Argument checks run before any
 * HIP call, so ATTN_EINVAL / ATTN_EUNSUPPORTED never touch the device.
 * libattn never prints and never exits.
 */
#ifndef LIBATTN_H
#define LIBATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_OK 0
/* null pointer, B/T/NH < 1, C < NH, C % NH != 0, causal not 0/1, misaligned
 * or overlapping buffers, or a tensor too large for 32-bit in-batch offsets
 * (T*3C >= 2^31, 64*3C*4 >= 2^32 bytes for one tile, or T*T >= 2^31 for the
 * materialised calls) */
#define ATTN_EINVAL (-1)
/* head size hs = C/NH not in {16, 32, 64, 128} */
#define ATTN_EUNSUPPORTED (-2)
/* a HIP call (workspace allocation, kernel launch) failed */
#define ATTN_EHIP (-3)

/*
 * Fused forward, fp32.  Writes out (B,T,C) and lse (B,NH,T).
 * causal = 1 masks keys j > t; causal = 0 attends to every key.
 */
int attn_forward(float* out, float* lse, const float* qkv,
                 int B, int T, int C, int NH, int causal);

/*
 * Fused backward, fp32.  Reads dout (B,T,C), qkv, and the forward's out and
 * lse; writes dqkv (B,T,3C) = [dq | dk | dv].  It runs a pre-pass that
 * forms D = rowsum(dout*out) and clears the dq third, then one kernel per
 * 64-key tile that recomputes the probabilities from lse, forms dV, dP, dS
 * = P*(dP - D) and dK, and adds the tile's share of dq = scale * dS K into
 * the dq third with float atomics (the stages attn_backward_prepare and
 * attn_backward_dkdvdq below; dq's last bits vary with the order of those
 * additions).  Memory is O(B*NH*T): the only scratch is D in the library
 * workspace.  The stages attn_backward_dq + attn_backward_dkdv compute the
 * same result without atomics, recomputing the probabilities and dP a
 * second time for dq; the dS block store stages further below trade O(T^2)
 * caller-owned memory for that recompute.
 */
int attn_backward(float* dqkv, const float* dout, const float* qkv,
                  const float* out, const float* lse,
                  int B, int T, int C, int NH, int causal);

/*
 * attn_backward without any allocation, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc.  Same arguments, kernels and result as
 * attn_backward (bit for bit for dk and dv; dq up to the order of its
 * atomic additions); its D scratch (B*NH*T floats) lives in a fixed device
 * array of 4194304 floats (16 MiB) that each GPU the library runs on holds
 * from library load until the process ends.  Shapes with B*NH*T above
 * that return ATTN_EINVAL before any HIP call.  The first call on a device
 * looks up the array's address there (hipGetSymbolAddress); make that first
 * call outside graph capture.  Every call on one GPU shares its array, so
 * calls that overlap in time on one GPU (different streams or threads)
 * race: serialise them, e.g. on one stream.  The array holds no state a
 * call depends on: D is written in full before it is read.
 */
int attn_backward_noalloc(float* dqkv, const float* dout, const float* qkv,
                          const float* out, const float* lse,
                          int B, int T, int C, int NH, int causal);

/*
 * The stages of attn_backward, for callers that want to time, order or
 * overlap them, or to own the D buffer (these calls allocate nothing).
 * D (B,NH,T) fp32 = dout . out per row and head (D[t] = sum_j att[t,j]
 * datt[t,j], the row term of the closed-form softmax gradient of
 * softmax_autoregressive_backward_kernel7 in llm.c
 * dev/cuda/attention_backward.cu); dq_t = scale * sum_j dS[t,j] k_j is the
 * dq product of attention_backward_cpu there.
 *   attn_backward_prepare: writes D and sets the dq third of dqkv to 0
 *       (the dk and dv thirds are not touched);
 *   attn_backward_dkdvdq: reads D, writes the dk and dv thirds of dqkv and
 *       ADDS each key tile's share of dq into the dq third (float atomics,
 *       so dq's last bits depend on their order).  The dq third must hold
 *       zeros, as attn_backward_prepare leaves it, or the dq to add to.
 *       dqkv must be ordinary device memory of the GPU the call runs on
 *       (hipMalloc, as torch allocates it): the hardware float atomics are
 *       not defined on host-mapped or fine-grained memory.  The same holds
 *       for attn_backward and attn_backward_noalloc.
 * attn_backward runs prepare then dkdvdq on the same stream.  The recompute
 * order, deterministic and free of atomics:
 *   attn_backward_dq: writes D and the dq third of dqkv (it recomputes the
 *       probabilities and dP itself);
 *   attn_backward_dkdv: reads that D, writes the dk and dv thirds of dqkv.
 * attn_backward_preprocess computes D alone (the same value the other calls
 * write, up to summation order), for callers that run dkdv first or need D
 * by itself.
 */
int attn_backward_prepare(float* dqkv, float* D, const float* dout, const float* out,
                          int B, int T, int C, int NH);
int attn_backward_dkdvdq(float* dqkv, const float* dout, const float* qkv,
                         const float* lse, const float* D,
                         int B, int T, int C, int NH, int causal);
int attn_backward_preprocess(float* D, const float* dout, const float* out,
                             int B, int T, int C, int NH);
int attn_backward_dq(float* dqkv, float* D, const float* dout, const float* qkv,
                     const float* out, const float* lse,
                     int B, int T, int C, int NH, int causal);
int attn_backward_dkdv(float* dqkv, const float* dout, const float* qkv,
                       const float* lse, const float* D,
                       int B, int T, int C, int NH, int causal);

/*
 * The dS block store stages of the fp32 backward.  dS[t,j] = att[t,j] *
 * (datt[t,j] - D[t]) (unscaled: dpreatt = scale * dS) is the closed-form
 * softmax gradient of softmax_autoregressive_backward_kernel7 in llm.c
 * dev/cuda/attention_backward.cu; dq_t = scale * sum_j dS[t,j] k_j is the
 * dq product of attention_backward_cpu there.  Storing dS once, while the
 * dK/dV kernel has it, saves the dQ kernel two of its three fp32
 * contractions (recomputing S and dP).
 *   attn_backward_ds_bytes: bytes of the dS block store for this shape: one
 *       64x64 fp32 block per (64-query tile, 64-key tile) pair the mask
 *       keeps (the lower triangle of tiles when causal, all of them
 *       otherwise), per head.  B*NH*ntile*(ntile+1)/2*16 KiB causal, ntile =
 *       ceil(T/64).  Returns 0 for arguments the other calls would reject.
 *   attn_backward_dkdv_ds: as attn_backward_dkdv (reads D from
 *       attn_backward_preprocess), and also writes every block of dS into
 *       dS (caller-owned device memory of attn_backward_ds_bytes bytes; its
 *       layout is internal to libattn and only attn_backward_dq_ds reads it).
 *   attn_backward_dq_ds: reads dS written by attn_backward_dkdv_ds for the
 *       same shape and qkv, writes the dq third of dqkv.
 * Neither allocates.  Errors as for the other calls (dS is checked like any
 * tensor argument: non-null, 16-byte aligned, no overlap).
 */
uint64_t attn_backward_ds_bytes(int B, int T, int C, int NH, int causal);
int attn_backward_dkdv_ds(float* dqkv, float* dS, const float* dout, const float* qkv,
                          const float* lse, const float* D,
                          int B, int T, int C, int NH, int causal);
int attn_backward_dq_ds(float* dqkv, const float* dS, const float* qkv,
                        int B, int T, int C, int NH, int causal);

/*
 * Fused forward and backward with bfloat16 inputs and outputs and fp32
 * accumulation (the mixed-precision scheme of "LLM Systems 10 & 11:
 * Accelerating Transformer Training and Inference", section 1: low-precision
 * operands, higher-precision accumulation).  lse stays fp32.  Probabilities
 * and dS are rounded to bf16 only as matrix-core operands.
 * attn_backward_bf16 (and attn_backward_f16) runs the dQ stage, which writes
 * D to the workspace, then the dK/dV stage; for short sequences (T <= 256
 * with hs = 16, 128 < T <= 256 with hs = 32 or 64) it runs instead one
 * kernel with one workgroup per head that keeps the head's dS on chip, forms
 * D itself and uses no workspace.  Both give the same quantities to within
 * the rounding of dS and of the fp32 sums; each is deterministic.
 */
int attn_forward_bf16(uint16_t* out, float* lse, const uint16_t* qkv,
                      int B, int T, int C, int NH, int causal);
int attn_backward_bf16(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                       const uint16_t* out, const float* lse,
                       int B, int T, int C, int NH, int causal);
/* bf16 versions of the backward stages (D stays fp32). */
int attn_backward_preprocess_bf16(float* D, const uint16_t* dout, const uint16_t* out,
                                  int B, int T, int C, int NH);
int attn_backward_dq_bf16(uint16_t* dqkv, float* D, const uint16_t* dout, const uint16_t* qkv,
                          const uint16_t* out, const float* lse,
                          int B, int T, int C, int NH, int causal);
int attn_backward_dkdv_bf16(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                            const float* lse, const float* D,
                            int B, int T, int C, int NH, int causal);

/*
 * Split-KV forward (16-bit path), for shapes whose plain forward grid leaves
 * the chip under-filled (few heads per GPU at long T: e.g. 2 heads of
 * T = 8192 give 128 query tiles for 256 compute units).  The keys each
 * query tile sees are split into chunks of kv_chunk keys, one workgroup per
 * (query tile, chunk); each writes its output normalised over its own keys
 * and that range's log-sum-exp, and a merge forms, per row,
 * L = log sum_p exp(lse_p), out = sum_p exp(lse_p - L) o_p: the rescale the
 * running softmax applies from one key block to the next ("Umakini wa
 * kujitegemea, kerneli za CUDA na FlashAttention", the FlashAttention part),
 * applied across workgroups.  Same out and lse as attn_forward_bf16 / _f16
 * up to rounding (the partial outputs stay fp32; out is rounded once).
 *   kv_chunk: keys per chunk, a positive multiple of 64, or 0 for the
 *       library's choice (attn_forward_splitkv_chunk: the longest
 *       power-of-two number of 64-key tiles that keeps a workgroup per
 *       compute unit; T rounded up to 64, i.e. no split, when the unsplit
 *       grid already does).  Returns the chunk in keys or a negative status.
 *   work: caller-owned device memory of attn_forward_splitkv_bytes bytes
 *       (fp32 partial outputs and log-sum-exps of every chunk, layout
 *       internal); 0 bytes when the chunk covers all keys, in which case
 *       the plain forward runs and work is not touched (it must still be a
 *       valid, aligned, non-null pointer).  attn_forward_splitkv_bytes
 *       returns 0 also for arguments the other calls would reject.
 * Nothing is allocated.  Errors as for attn_forward_bf16, plus ATTN_EINVAL
 * for a kv_chunk that is negative or not a multiple of 64.
 */
int attn_forward_splitkv_chunk(int B, int T, int C, int NH, int causal);
uint64_t attn_forward_splitkv_bytes(int B, int T, int C, int NH, int causal, int kv_chunk);
int attn_forward_splitkv_bf16(uint16_t* out, float* lse, const uint16_t* qkv, float* work,
                              int B, int T, int C, int NH, int causal, int kv_chunk);
int attn_forward_splitkv_f16(uint16_t* out, float* lse, const uint16_t* qkv, float* work,
                             int B, int T, int C, int NH, int causal, int kv_chunk);

/*
 * Split backward (16-bit path), the counterpart of the split-KV forward for
 * under-filled grids.  The dQ kernel's keys and the dK/dV kernel's queries
 * are split into chunks of kv_chunk (keys, resp. query rows), one workgroup
 * per (tile, chunk); each writes its fp32 partial sum of dq, resp. dk and
 * dv (the sums over key or query ranges of the analytic backward of
 * attention_backward_cpu in llm.c dev/cuda/attention_backward.cu, with the
 * softmax step of its kernel 7), and a last kernel adds the partials of
 * every row in a fixed order and rounds once to the 16-bit type, so the
 * result is deterministic.  Same dqkv as attn_backward_bf16 / _f16 up to
 * rounding.
 *   kv_chunk: as for attn_forward_splitkv_bf16 (0: the library's choice).
 *   work: caller-owned device memory of attn_backward_splitkv_bytes bytes:
 *       D (B*NH*T floats, rounded up to 64) and, when the chunk splits the
 *       keys, fp32 partial sums (3*ceil(T/kv_chunk)*B*T*C floats).  Without
 *       a split the call runs attn_backward_dq_bf16 / _f16 and
 *       attn_backward_dkdv_bf16 / _f16 with D in work.
 * Nothing is allocated.  Errors as for attn_forward_splitkv_bf16.
 */
uint64_t attn_backward_splitkv_bytes(int B, int T, int C, int NH, int causal, int kv_chunk);
int attn_backward_splitkv_bf16(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                               const uint16_t* out, const float* lse, float* work,
                               int B, int T, int C, int NH, int causal, int kv_chunk);
int attn_backward_splitkv_f16(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                              const uint16_t* out, const float* lse, float* work,
                              int B, int T, int C, int NH, int causal, int kv_chunk);

/*
 * The same fused forward, backward and backward stages with IEEE half
 * (fp16) tensors, passed as uint16_t bit patterns: the section names FP16
 * beside BF16 for mixed-precision training.  Same kernels, fp16 matrix-core
 * operands, fp32 accumulation, round to nearest even on output; lse and D
 * stay fp32.  fp16 keeps 3 more mantissa bits than bf16 but its range ends
 * at 65504: out, dS and the gradients must stay inside it.
 */
int attn_forward_f16(uint16_t* out, float* lse, const uint16_t* qkv,
                     int B, int T, int C, int NH, int causal);
int attn_backward_f16(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                      const uint16_t* out, const float* lse,
                      int B, int T, int C, int NH, int causal);
int attn_backward_preprocess_f16(float* D, const uint16_t* dout, const uint16_t* out,
                                 int B, int T, int C, int NH);
int attn_backward_dq_f16(uint16_t* dqkv, float* D, const uint16_t* dout, const uint16_t* qkv,
                         const uint16_t* out, const float* lse,
                         int B, int T, int C, int NH, int causal);
int attn_backward_dkdv_f16(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                           const float* lse, const float* D,
                           int B, int T, int C, int NH, int causal);

/*
 * Fused forward with 8-bit floating-point q, k, v ("LLM Systems 10 & 11:
 * Accelerating Transformer Training and Inference", section 1.3,
 * Mixed-precision Calculation, which names FP8 beside FP16 for the forward
 * and backward).  qkv holds OCP FP8 E4M3 bytes (sign, 4 exponent bits with
 * bias 7, 3 mantissa bits; largest finite magnitude 448; 0x7F and 0xFF are
 * NaN), packed (B, T, 3C) like the other calls.  Every product accumulates
 * in fp32 and the softmax runs in fp32; the probabilities enter the P V
 * product rounded to E4M3 (round to nearest even; below 2^-10 of a row's
 * running maximum they become 0), and the row sums are taken over the same
 * rounded values.  out is bfloat16 (B, T, C), round to nearest even; lse is
 * fp32 (B, NH, T) as for attn_forward.  Forward only: the backward runs in
 * bf16 or fp16 (attn_backward_bf16 / _f16 with a 16-bit copy of qkv).
 * Requirements and errors as for attn_forward_bf16 (qkv 16-byte aligned).
 * Nothing is allocated.
 */
int attn_forward_fp8(uint16_t* out, float* lse, const uint8_t* qkv,
                     int B, int T, int C, int NH, int causal);

/*
 * Materialised forward, fp32, as the pages' reference does it: writes the
 * full unscaled preatt = q.k (B,NH,T,T) including masked entries, att
 * (B,NH,T,T) with masked entries exactly 0, and out (B,T,C).
 * (llm.c attention_backward.cu: attention_forward_cpu and the
 * permute / sgemm / softmax / sgemm / unpermute GPU sequence.)
 */
int attn_forward_materialized(float* out, float* preatt, float* att, const float* qkv,
                              int B, int T, int C, int NH, int causal);

/*
 * Materialised backward, fp32, from the forward's att: writes datt = dout.v
 * (dense, every (t,j)), dpreatt (exactly 0 on masked entries) and dqkv.
 * With causal = 1 only the lower triangle of att is read (entries above the
 * diagonal are taken as 0).  Needs no workspace.
 * (llm.c attention_backward.cu: attention_backward_cpu and
 * softmax_autoregressive_backward_kernel7.)
 */
int attn_backward_materialized(float* dqkv, float* dpreatt, float* datt,
                               const float* dout, const float* qkv, const float* att,
                               int B, int T, int C, int NH, int causal);

/*
 * Decode, fp32: attention of the last query row t = T-1 of every sequence
 * and head against all of its keys 0..T-1 (the causal row T-1, which is also
 * the non-causal one) -- one step of autoregressive inference over the
 * packed qkv of the T tokens so far, the same computation with a single
 * query row ("LLM Systems 10 & 11: Accelerating Transformer Training and
 * Inference", section 2).  Reads only row T-1 of q and rows 0..T-1 of k, v.
 * Writes out (B, C) = [b, h*hs+i] and lse (B, NH).  The keys are split into
 * ranges of 128 or 256 per workgroup and the partial results merged as
 * attn_merge does; the partials live in the library workspace (at most
 * ceil(T/128) * B * (C + NH) floats).
 */
int attn_decode(float* out, float* lse, const float* qkv, int B, int T, int C, int NH);

/* Decode with bf16 qkv and out (fp32 arithmetic, fp32 lse). */
int attn_decode_bf16(uint16_t* out, float* lse, const uint16_t* qkv, int B, int T, int C,
                     int NH);

/* Decode with fp16 (IEEE half) qkv and out (fp32 arithmetic, fp32 lse). */
int attn_decode_f16(uint16_t* out, float* lse, const uint16_t* qkv, int B, int T, int C,
                    int NH);

/*
 * Merge of partial attention results over disjoint key sets: the rescale
 * the online softmax applies between key tiles (FlashAttention part of
 * "Umakini wa kujitegemea, kerneli za CUDA na FlashAttention"), applied
 * across parts.  Part p gives o_parts[p] (B, T, C) fp32, normalised over its
 * own keys, and lse_parts[p] (B, NH, T) (natural log, scaled domain; -inf for
 * a row with no key in the part).  Writes
 *     lse = log sum_p exp(lse_p),   out = sum_p exp(lse_p - lse) o_p,
 * and out = 0, lse = -inf where every part is empty.  o_parts is
 * (nparts, B, T, C) and lse_parts (nparts, B, NH, T), contiguous; nparts >= 1.
 * Needs no workspace.
 */
int attn_merge(float* out, float* lse, const float* o_parts, const float* lse_parts, int nparts,
               int B, int T, int C, int NH);

/* Merge with a bf16 out (parts and lse stay fp32). */
int attn_merge_bf16(uint16_t* out, float* lse, const float* o_parts, const float* lse_parts,
                    int nparts, int B, int T, int C, int NH);

/* Merge with an fp16 out (parts and lse stay fp32). */
int attn_merge_f16(uint16_t* out, float* lse, const float* o_parts, const float* lse_parts,
                   int nparts, int B, int T, int C, int NH);

/*
 * LayerNorm over the rows of inp (N, C), row-major: the normalisation of
 * "llm.c 的中文注解-20240423", section 1.8, with the single-reduction
 * forward and backward of "LLM Systems 10 & 11: Accelerating Transformer
 * Training and Inference", section 1.2.1.  Per row r:
 *     mean[r] = sum_c x[r,c] / C,   var = sum_c (x[r,c] - mean[r])^2 / C,
 *     rstd[r] = 1 / sqrt(var + 1e-5),
 *     out[r,c] = (x[r,c] - mean[r]) * rstd[r] * weight[c] + bias[c].
 * out and inp are (N, C); mean and rstd are (N,) fp32 (kept for the
 * backward); weight and bias are (C,) fp32.  Every pointer is a
 * caller-owned device pointer, 16-byte aligned; outputs may not overlap
 * each other or an input.  N, C >= 1 (any C; rows of C % 4 == 0 use vector
 * loads).  No workspace.  Errors: ATTN_EINVAL for a NULL or misaligned
 * pointer, N or C < 1, or overlapping buffers; ATTN_EHIP for a launch
 * failure.
 */
int layernorm_forward(float* out, float* mean, float* rstd, const float* inp, const float* weight,
                      const float* bias, int N, int C);

/* LayerNorm with bfloat16 out and inp (round to nearest even); mean, rstd,
 * weight, bias and all arithmetic fp32. */
int layernorm_forward_bf16(uint16_t* out, float* mean, float* rstd, const uint16_t* inp,
                           const float* weight, const float* bias, int N, int C);

/*
 * Gradients of layernorm_forward, written (=):
 *     xhat = (x - mean) * rstd,  g = weight * dout,
 *     dinp[r,c]  = rstd[r] * (g[r,c] - sum_c g[r,:] / C - xhat[r,c] * sum_c (g * xhat)[r,:] / C),
 *     dweight[c] = sum_r dout[r,c] * xhat[r,c],   dbias[c] = sum_r dout[r,c],
 * with mean and rstd as layernorm_forward wrote them for the same inp.
 * dinp, dout and inp are (N, C); dweight, dbias and weight (C,); mean and
 * rstd (N,).  Uses the library workspace (2 * C floats per chunk of 16
 * rows) for partial column sums, which are added in a fixed order: results
 * are bitwise deterministic.  Errors as layernorm_forward, plus ATTN_EHIP
 * if the workspace cannot be allocated.
 */
int layernorm_backward(float* dinp, float* dweight, float* dbias, const float* dout,
                       const float* inp, const float* weight, const float* mean, const float* rstd,
                       int N, int C);

/* The backward with bfloat16 dinp, dout and inp; the rest as above. */
int layernorm_backward_bf16(uint16_t* dinp, float* dweight, float* dbias, const uint16_t* dout,
                            const uint16_t* inp, const float* weight, const float* mean,
                            const float* rstd, int N, int C);

/* LayerNorm with IEEE-half out and inp (round to nearest even), the 16-bit
 * storage with fp32 accumulation that "LLM Systems 10 & 11: Accelerating
 * Transformer Training and Inference" (section 1.2.1) names; the rest as
 * layernorm_forward.  Outputs must stay below 65504 in magnitude. */
int layernorm_forward_f16(uint16_t* out, float* mean, float* rstd, const uint16_t* inp,
                          const float* weight, const float* bias, int N, int C);

/* The backward with IEEE-half dinp, dout and inp; the rest as
 * layernorm_backward. */
int layernorm_backward_f16(uint16_t* dinp, float* dweight, float* dbias, const uint16_t* dout,
                           const uint16_t* inp, const float* weight, const float* mean,
                           const float* rstd, int N, int C);

/* Set the HIP stream (a hipStream_t, or NULL for the null stream) used by
 * the calling thread's subsequent calls.  Always returns ATTN_OK. */
int attn_set_stream(void* hip_stream);

/* Message describing the calling thread's last non-OK status ("" if none).
 * The string stays valid until the thread's next libattn call. */
const char* attn_last_error(void);

/* Free the workspace on every device it was allocated on.  Must
 * not race with work still queued that uses it (synchronise first). */
void attn_release(void);

/*
 * The projections on either side of the attention block, on the matrix
 * cores with the elementwise steps fused into the product's store (the
 * kernel fusion of "LLM Systems 10 & 11: Accelerating Transformer Training
 * and Inference", section 1).  Row-major, fp32 accumulation:
 *
 *   attn_qkv_projection:  qkv[m][n] = sum_k x[m][k] w[n][k] + bias[n]
 *   attn_out_projection:  y[m][n]   = sum_k a[m][k] w[n][k] + bias[n] + residual[m][n]
 *
 * The QKV projection is Q = X W_Q, K = X W_K, V = X W_V of "Umakini wa
 * kujitegemea, kerneli za CUDA na FlashAttention" (section 1) for all heads
 * at once: with M = B*T rows of x (C = K wide) and w of shape (N = 3C, K)
 * whose rows are the columns of [W_Q | W_K | W_V] (the layout in which
 * each output column's weights are contiguous), qkv is the packed
 * (B, T, 3C) input of attn_forward.  The output projection adds the
 * residual stream as residual_forward_kernel does ("llm.c 的中文注解-20240423",
 * section 1.15: out = inp1 + inp2), here in the same pass.
 *   x, a (M, K); w (N, K); bias (N) fp32; residual, y, qkv (M, N).
 *   _bf16: x, a, w, residual and the output bf16, bias fp32; the output
 *   is rounded once (to nearest even) from the fp32 sum.
 * Errors: ATTN_EINVAL for a null or misaligned pointer, M, K or N < 1,
 * K not a multiple of 4 (fp32) or 8 (bf16), N not a multiple of 4, K too
 * large for 32-bit tile offsets, or an output overlapping an input.
 * Nothing is allocated.
 */
int attn_qkv_projection(float* qkv, const float* x, const float* w, const float* bias,
                        int M, int K, int N);
int attn_qkv_projection_bf16(uint16_t* qkv, const uint16_t* x, const uint16_t* w,
                             const float* bias, int M, int K, int N);
int attn_out_projection(float* y, const float* a, const float* w, const float* bias,
                        const float* residual, int M, int K, int N);
int attn_out_projection_bf16(uint16_t* y, const uint16_t* a, const uint16_t* w,
                             const float* bias, const uint16_t* residual, int M, int K, int N);

#ifdef __cplusplus
}
#endif

#endif /* LIBATTN_H */
