/*
 * nucleus.h -- C ABI of libnucleus, batched top-p (nucleus) sampling over
 * full-vocabulary logits on AMD Instinct MI355X (gfx950).
 *
 * One call samples one token for each of B rows of logits.  Each row carries
 * its own temperature T, min-p, top-k and top-p, applied as one chain:
 *
 *   temperature -> min-p -> top-k -> top-p -> renormalise -> sample
 *
 * (the order named in "What do temperature, top-k and top-p each do to the
 * next-token distribution, and in what order does a serving engine apply
 * them?", TL;DR and reference sampler).  Per row b with logits x:
 *
 *  - Temperature divides the logits before the softmax: p_i is proportional
 *    to exp((x_i - max x)/T) (the tempered-softmax equation of that page).
 *    T <= 0 is greedy: the lowest index among the maximal logits ("Implement
 *    batched top-p sampling with temperature", "A strong answer" and "Why
 *    each line is there", item 4).
 *  - min-p drops token i iff p_i < min_p * max_j p_j (reference sampler of the
 *    order page).  min_p <= 0 is off; min_p > 1 acts as 1.
 *  - top-k keeps the tokens whose logit is >= the k-th largest remaining
 *    logit; ties at the k-th value survive (order page, reference sampler and
 *    its edge-case note).  k <= 0 is off; k >= the number of remaining tokens
 *    is a no-op.
 *  - top-p keeps token i iff the probability mass of the remaining tokens
 *    strictly more probable than i is < p, measured on the distribution left
 *    by min-p and top-k, renormalised.  Tokens tied at the cut share a fate,
 *    the most probable level is always kept, p >= 1 keeps every remaining
 *    token and p <= 0 keeps only the most probable level ("Top-p (Nucleus)
 *    Sampling, in depth", "Batched top-p with a different p per request" and
 *    "Boundaries and ties"; "Implement batched top-p sampling ...", "How to
 *    approach it").
 *  - The kept set is renormalised and one token is drawn by the exponential
 *    race argmax_i p_i / E_i, E_i ~ Exp(1) (order page, "A strong answer",
 *    last paragraph), lowest index on exact ties.  E_i = -ln u_i,
 *    u_i = (r_i + 1/2) / 2^32, where r_i is word (i mod 4) of
 *    Philox4x32-10 (Salmon et al., SC'11) with key (seed low 32 bits, seed
 *    high 32 bits) and counter (i / 4, b, step low 32 bits, step high
 *    32 bits).  The draw of row b depends only on (seed, step, b) and row b's
 *    own inputs.
 *  - A row with a NaN or +inf logit, no finite logit, or a NaN T / top-p /
 *    min-p is a row error ("Top-p (Nucleus) Sampling, in depth", "Failure
 *    modes": check for NaN and fail the request).  -inf logits are masked
 *    tokens: probability 0, never kept.
 *
 * Threading: calls are asynchronous on the given stream and never
 * synchronise the device.  Calls on different streams need distinct
 * workspaces.  The library keeps no pointer after a call returns.
 */
#ifndef NUCLEUS_H
#define NUCLEUS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes.  Argument errors are detected on the host before anything is
 * launched; nothing is written in that case. */
#define NUCLEUS_OK 0
#define NUCLEUS_EINVAL (-1)     /* null required pointer, B < 0, V < 1, V >= 2^31, bad dtype,
                                   stride < V, or a pointer not aligned to its element size */
#define NUCLEUS_EWORKSPACE (-2) /* workspace missing or smaller than nucleus_workspace_bytes() */
#define NUCLEUS_ELAUNCH (-3)    /* the HIP runtime refused a launch */
#define NUCLEUS_EDEVICE (-4)    /* no usable gfx950 device for the current HIP context */

/* Option flags. */
#define NUCLEUS_FLAG_SINGLE_WORKGROUP 1 /* run every row, every phase, on one workgroup that
                                           streams the row from memory once per phase (the path
                                           every batch takes by default but small batches of
                                           long rows, below); no
                                           workspace needed.  Same results, bit for bit.  For
                                           verification and for callers that cannot provide a
                                           workspace. */
#define NUCLEUS_FLAG_SPLIT_ROWS 2       /* split every row over register-resident workgroups
                                           (the path taken by default by batches of B < 128
                                           rows of V > 32768 tokens with B * ceil(V / 8192)
                                           <= 1536)
                                           whatever the batch size; rows longer than 64 * 8192
                                           tokens are then NUCLEUS_EINVAL.  Same results, bit
                                           for bit.  For verification. */
#define NUCLEUS_FLAG_ROW_RACE 4         /* one workgroup per row for the histogram passes and the
                                           race spread over 8192-token chunks of all rows,
                                           whatever the batch size (needs a workspace: 256 bytes
                                           plus a 64 KB candidate list per row).  Same results,
                                           bit for bit. */

/* Logit element types. */
#define NUCLEUS_F32 0
#define NUCLEUS_BF16 1

typedef struct nucleus_options {
    int32_t dtype;               /* NUCLEUS_F32 (default) or NUCLEUS_BF16 */
    int32_t flags;               /* 0, or one NUCLEUS_FLAG_* value (not both) */
    void* stream;                /* hipStream_t to launch on; NULL = the null stream */
    int64_t row_stride;          /* elements between row starts; 0 means V */
    void* workspace;             /* device scratch of >= nucleus_workspace_bytes(B, V, dtype) bytes,
                                    256-byte aligned, owned by the caller; may be NULL when that
                                    size is 0.  Its contents need no initial value and may be
                                    reused by any later call.  Calls that may overlap (different
                                    streams) need different workspaces. */
    size_t workspace_bytes;      /* size of workspace */
    float* out_min_kept_logit;   /* optional device [B]: the smallest kept logit (NaN on a row
                                    error).  For T > 0 rows the kept set is exactly
                                    {i : x_i finite and x_i >= out_min_kept_logit[b]};
                                    for greedy rows it is {out_token[b]}. */
    /* Since version 210 (a caller built against an older header zero-fills
     * them when it zero-initialises the struct): */
    const uint64_t* seeds;       /* optional device [B]: per-request Philox keys; row b then
                                    draws with key (lo, hi 32 bits of seeds[b]) instead of
                                    the call's seed, so its draw does not depend on the rest
                                    of the batch ("Top-p (Nucleus) Sampling, in depth",
                                    "Logprobs, speculative decoding and reproducibility").
                                    NULL: every row uses the call's seed. */
    float* out_logprobs;         /* optional device [B, V]: log-probabilities of the same
                                    processed distribution as out_probs (the same section):
                                    (x_i - m)/T - ln S_keep on kept tokens, -inf outside the
                                    nucleus; 0 / -inf for greedy rows; NaN on a row error.
                                    Finite for kept tokens whose probability underflows. */
    /* Since version 240: the pre-chain, applied to the raw logits before
     * everything above ("Top-p (Nucleus) Sampling, in depth", "Where top-p
     * sits in the sampler chain"; penalties on raw logits so they change the
     * greedy choice too, "What do temperature, top-k and top-p ...", "What
     * interviewers probe next").  With c_i the occurrences of token i in the
     * row's history, for c_i > 0:  y = x / rho if x > 0 else x * rho, then
     * x' = y - (a_f * c_i + a_p); then x' = -inf where the mask forbids i.
     * Each step is one fp32 operation in that order (no fused multiply-add).
     * The sampler (validation included) sees only x'.  Any of these fields
     * set selects the one-workgroup-per-row path (NUCLEUS_FLAG_SPLIT_ROWS and
     * NUCLEUS_FLAG_ROW_RACE are then NUCLEUS_EINVAL) and needs V <= 166912;
     * NULL / 0 leaves the logits as they are. */
    const int32_t* history;            /* optional device [B, history_len] int32: each row's earlier
                                          tokens, -1 padded (ids outside [0, V) are ignored) */
    int64_t history_len;               /* 0 .. 1024 */
    const float* repetition_penalty;   /* optional device [B]: rho (> 0; 1 = off) */
    const float* frequency_penalty;    /* optional device [B]: a_f (0 = off) */
    const float* presence_penalty;     /* optional device [B]: a_p (0 = off) */
    const uint32_t* allowed_mask;      /* optional device [B, ceil(V/32)] uint32: token i allowed iff
                                          bit (i mod 32) of word i / 32 is set (a grammar / JSON
                                          constraint) */
    /* Since version 260, for tests of the failure path only ("Top-p (Nucleus)
     * Sampling, in depth", "Failure modes": a failing request must not hang
     * the batch): */
    int64_t split_give_up_row;   /* 0: off.  r + 1 (r >= 0): on the split-row path the workgroups
                                    of row r give up every wait at once, as if the row's
                                    workgroups could not meet, so row r reports token -2 and
                                    every other row is sampled as usual.  Ignored by the other
                                    paths; negative is NUCLEUS_EINVAL. */
} nucleus_options;

/*
 * Sample one token per row.
 *
 * logits          device, [B, row_stride] elements of dtype, row-major; read only.
 *                 fp32 rows must start on 16-byte boundaries or the call uses the
 *                 (slower) unaligned path; bf16 rows are widened exactly to fp32.
 * B, V            batch rows and vocabulary size: B >= 0, 1 <= V < 2^31.
 *                 B == 0 returns NUCLEUS_OK and launches nothing.
 * temperature     device [B] float, required.
 * top_p           device [B] float, required.
 * top_k           device [B] int32, or NULL (top-k off for every row).
 * min_p           device [B] float, or NULL (min-p off for every row).
 * seed, step      Philox key and the high counter words; reusing them reproduces
 *                 the draws exactly.
 * out_token       device [B] int32: the sampled id, or -1 on a row error (-2 if, on the
 *                 split-row path, the workgroups of a row could not meet within
 *                 seconds, e.g. because other work held the whole device; that row's
 *                 other outputs are then not written, and the other rows are unaffected).
 * out_keep_count  device [B] int32: size of the kept set (1 for greedy rows,
 *                 0 on a row error).
 * out_probs       device [B, V] float, or NULL: the renormalised kept
 *                 distribution (one-hot for greedy rows, zeros on a row error).
 * opt             NULL for all defaults (fp32, null stream, no stride, no workspace).
 *
 * Returns NUCLEUS_OK or a negative code; the outputs are complete once the
 * stream reaches the call.  All device buffers are owned by the caller and
 * must stay valid until then.
 */
int nucleus_sample(const void* logits, int64_t B, int64_t V, const float* temperature,
                   const float* top_p, const int32_t* top_k, const float* min_p, uint64_t seed,
                   uint64_t step, int32_t* out_token, int32_t* out_keep_count, float* out_probs,
                   const nucleus_options* opt);

/*
 * nucleus_sample for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, results and return codes as nucleus_sample, except that the
 * scratch the chosen path needs (the split-row and row-race paths; the
 * one-workgroup-per-row path needs none) comes from a static device array of
 * nucleus_noalloc_scratch_bytes() bytes (32 MiB) that the library holds on
 * every GPU it runs on until the process ends; opt->workspace and
 * opt->workspace_bytes are ignored.  Returns NUCLEUS_EWORKSPACE, launching
 * nothing, when the call's path needs more scratch than that (for example
 * B = 127 rows of 524288 tokens on the split-row path); NUCLEUS_EDEVICE if
 * the runtime cannot give the array's address.  Makes no device allocation.
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (different streams, or other threads) race and give undefined
 * results.  The array needs no initial value: each call tags its
 * synchronisation words with a value of its own.
 */
int nucleus_sample_noalloc(const void* logits, int64_t B, int64_t V, const float* temperature,
                           const float* top_p, const int32_t* top_k, const float* min_p, uint64_t seed,
                           uint64_t step, int32_t* out_token, int32_t* out_keep_count, float* out_probs,
                           const nucleus_options* opt);

/* Size in bytes of nucleus_sample_noalloc's static scratch on each GPU. */
size_t nucleus_noalloc_scratch_bytes(void);

/*
 * Sample one token per row by sort-free rejection ("Top-p (Nucleus) Sampling,
 * in depth", "Sort-free top-p by rejection sampling"): a second algorithm for
 * the chain above without top-k (temperature -> min-p -> top-p -> sample),
 * which finds no cut.  Per row, a pivot starts below every logit; each round
 * proposes the race winner argmax_i e_i / E_i over the finite tokens above
 * the pivot, with the same Philox words E_i as nucleus_sample, and accepts it
 * iff it survives min-p and it is in the top level, or p >= 1, or the mass of
 * the surviving tokens strictly more probable than it is below p (measured
 * on the survivors, renormalised).  A rejected proposal becomes the pivot.
 * Reusing the words is a valid draw (an exponential race restricted to the
 * tokens above the pivot proposes in proportion to their weights, whatever
 * was rejected before), and the accepted token is the first kept token in
 * race order: the token nucleus_sample draws with the same seed, step and
 * parameters (top_k NULL), up to rows within rounding of a boundary.
 *
 * logits, B, V, temperature, top_p, min_p, seed, step: as for nucleus_sample.
 * out_token   device [B] int32: the accepted id; the lowest-index argmax for
 *             T <= 0; -1 on a row error (as nucleus_sample) or if no
 *             proposal was accepted within 64 rounds (a row needs at most one
 *             round per distinct logit value; typical rows need 1 or 2).
 * out_rounds  device [B] int32, or NULL: rounds run (0 for greedy and error
 *             rows, 64 when none was accepted).
 * opt         NULL, or options with dtype, stream, row_stride and seeds used;
 *             flags must be 0 and out_min_kept_logit and out_logprobs NULL
 *             (NUCLEUS_EINVAL otherwise); the workspace is not used.
 *
 * Returns NUCLEUS_OK or a negative code, with nucleus_sample's argument rules.
 * A row costs two passes over its logits per round (the first round's race
 * shares the pass that finds the max).
 */
int nucleus_sample_rejection(const void* logits, int64_t B, int64_t V, const float* temperature,
                             const float* top_p, const float* min_p, uint64_t seed, uint64_t step,
                             int32_t* out_token, int32_t* out_rounds, const nucleus_options* opt);

/*
 * Speculative-decoding acceptance against the truncated target ("Top-p
 * (Nucleus) Sampling, in depth", "Logprobs, speculative decoding and
 * reproducibility").  Per row b, the draft token d = draft_token[b], drawn
 * from the draft's own sampling distribution q (including any truncation the
 * draft applied), is accepted with probability min(1, p(d)/q(d)); otherwise
 * the token is drawn from the normalised positive part of p - q.  p must be
 * the target's truncated, renormalised distribution -- nucleus_sample's
 * out_probs for the target logits -- not its raw softmax; the output then
 * follows p exactly, whatever q is.
 *
 * Noise: the row's Philox key (seed, or opt->seeds[b]) with counter
 * (c0, b + 2^31, step low, step high): never the words nucleus_sample uses
 * for the same seed and step.  u = (r + 1/2) 2^-32 with r word 0 at
 * c0 = 0xFFFFFFFF decides acceptance: u q(d) < p(d).  The residual draw is
 * the exponential race argmax_i (p_i - q_i) / E_i over p_i > q_i, E_i from
 * word i mod 4 at c0 = i / 4, lowest index on ties.
 *
 * target_probs  device [B, V] float, rows contiguous: p.
 * draft_probs   device [B, V] float, rows contiguous: q.
 * draft_token   device [B] int32.
 * out_token     device [B] int32: d if accepted, else the residual draw; -1 if
 *               d is outside [0, V) or p - q has no positive entry (a target
 *               row error leaves p all zero).
 * out_accepted  device [B] int32, or NULL: 1 if the draft token was accepted.
 * opt           required for B > 0: stream, seeds and the workspace (at least
 *               nucleus_spec_workspace_bytes(B, V) bytes, 256-byte aligned,
 *               no initial value needed; NUCLEUS_EWORKSPACE otherwise) are
 *               used; dtype must be NUCLEUS_F32, row_stride 0 or V, flags 0,
 *               out_min_kept_logit and out_logprobs NULL (NUCLEUS_EINVAL
 *               otherwise).
 *
 * Returns NUCLEUS_OK or a negative code.  Asynchronous on opt->stream; calls
 * that may overlap need different workspaces.  An accepted row reads two
 * floats; a rejected row reads its p and q rows once, in 8192-token chunks
 * spread over the device.
 */
int nucleus_spec_verify(const float* target_probs, const float* draft_probs, const int32_t* draft_token,
                        int64_t B, int64_t V, uint64_t seed, uint64_t step, int32_t* out_token,
                        int32_t* out_accepted, const nucleus_options* opt);

/* Device workspace, in bytes, that nucleus_spec_verify needs: 8 bytes per
 * 8192-token chunk of every row.  0 for invalid shapes. */
size_t nucleus_spec_workspace_bytes(int64_t B, int64_t V);

/* Device workspace, in bytes, that nucleus_sample needs for a batch of this
 * shape and dtype with no flags: batches that split their rows by default
 * (B < 128, 32768 < V <= 64 * 8192, B * ceil(V / 8192) <= 1536) need the
 * split-row path's (per row: a 128-byte control block, 12.3 KB per
 * 8192-token chunk and a 64 KB candidate list); other batches need none.
 * Returns 0 for B == 0 and for invalid shapes. */
size_t nucleus_workspace_bytes(int64_t B, int64_t V, int32_t dtype);

/* The same for a call with the given option flags (0 for
 * NUCLEUS_FLAG_SINGLE_WORKGROUP; 0 for a flag combination nucleus_sample
 * rejects).  At most one flag may be set. */
size_t nucleus_workspace_bytes_for(int64_t B, int64_t V, int32_t dtype, int32_t flags);

/* Static description of a return code. */
const char* nucleus_strerror(int code);

/* Library version, major * 10000 + minor * 100 + patch. */
int nucleus_version(void);

/*
 * Read `bytes` bytes of device memory at `buf` once with 16-byte loads and
 * fold them into device `sink`, an array of 256 uint64 words (XOR-updated,
 * not cleared): the XOR of the 256 words changes by the XOR of the buffer's
 * little-endian 32-bit words, each of the last bytes % 16 bytes XORed in as
 * a value 0..255.  This is the HBM read ceiling the sampler's achieved
 * bandwidth is compared with.  `buf` must be 16-byte aligned.  Asynchronous
 * on `stream` (a hipStream_t, NULL = null stream).  Returns NUCLEUS_OK or a
 * negative code.
 */
int nucleus_stream_read(const void* buf, size_t bytes, uint64_t* sink, void* stream);

/*
 * Phase clocks, for profiling the one-workgroup-per-row path.  Only a library
 * built with NUCLEUS_PHASE_STAMPS (libnucleus_stamps.so) records them; the
 * product build returns NUCLEUS_EINVAL and records nothing.  After this call,
 * every nucleus_sample call with B <= rows that runs one workgroup per row
 * writes, for row b, the device's 100 MHz constant-rate clock at eight phase
 * boundaries to buf[16 b + k]: k = 0 start, 1 first pass (max, error flag,
 * fused histogram), 2 bins ready, 3 bin decision, 4 classification, 5 race
 * pass, 6 resolver and outputs, 7 probability pass (or its skip); and facts
 * about the row: buf[16 b + 8] its mode after the bin decision, + 9 the
 * crossing-bin candidates listed after the race pass, + 10 the marked runs
 * of 4-token groups that hold them (a run is one group in rows of up to
 * 2^18 groups).
 * A phase a row does not run leaves its word as it was.  buf: device,
 * [rows, 16] uint64, 8-byte aligned, owned by the caller and valid for every
 * later call; NULL turns the recording off.  Calls that overlap race on buf.
 */
int nucleus_phase_stamps(uint64_t* buf, int64_t rows);

#ifdef __cplusplus
}
#endif

#endif /* NUCLEUS_H */
