/*
 * adaln.h -- C ABI of the fused AdaLN (LayerNorm-Modulate) library for AMD
 * Instinct MI355X (gfx950).
 *
 * The operator is the one the AdaptiveLoad technical summary pages
 * (gist.science, arXiv 2605.17923) describe in section 2 ("Methodology"),
 * part B, "fused LayerNorm-Modulate kernels": each token row of x is
 * normalised over the feature dimension D and then modulated by per-sample
 * vectors, in one launch; in the backward pass the gradients of the
 * modulation parameters are reduced along the sequence dimension N over a
 * (d_tile, n_tile) grid with lanes pinned to features (the D-tile coalesced
 * reduction).  The formula, which the pages leave implicit, is read as:
 *
 *     mean = (1/D) sum_d x          var = (1/D) sum_d (x - mean)^2
 *     rstd = 1 / sqrt(var + 1e-6)   xhat = (x - mean) * rstd
 *     y    = xhat * (1 + scale[b]) + shift[b]
 *
 *     g      = dy * (1 + scale[b])
 *     dx     = rstd * (g - mean_d(g) - xhat * mean_d(g * xhat))
 *     dscale = sum_n dy * xhat      dshift = sum_n dy      (per b and d)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout.  Row-major, contiguous.  x, y, dy, dx are [B, N, D] in `dtype`;
 *   scale and shift are [B, D] in `dtype`; mean and rstd are [B, N] float32;
 *   dscale and dshift are [B, D] float32.  Row r = b*N + n.
 * dtype.  ADALN_F32 or ADALN_BF16.  Arithmetic is float32 in registers;
 *   bfloat16 outputs are rounded to nearest even.
 * Pointers.  Device pointers (hipMalloc'd or torch CUDA/HIP tensors), each
 *   16-byte aligned.  A pointer may be NULL only when its tensor has zero
 *   elements.  Input and output buffers must not overlap.
 * Sizes.  B, N >= 0; D > 0 and a multiple of 8 (bf16) or 4 (f32), at most
 *   adaln_max_d(dtype); B*N < 2^31 rows, B*D < 2^31.
 * Ownership.  The caller owns every buffer, including the backward
 *   workspace.  The library allocates no device memory and keeps no state
 *   between calls, so calls on different streams may run concurrently as long
 *   as they use distinct output and workspace buffers.
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the default
 *   stream).  Calls enqueue kernels on the calling thread's current HIP
 *   device, which must own the stream and every buffer, and return without
 *   synchronising.  Nothing is allocated, no memory is set with memset
 *   nodes and nothing waits, so the calls can be captured in a HIP graph.
 * Errors.  Arguments are validated on the host before any HIP call; a failing
 *   check returns a negative code and enqueues nothing.  A launch failure
 *   returns ADALN_ERR_HIP.  adaln_strerror() names a code; adaln_last_error()
 *   gives the calling thread's message for its most recent failing call.
 */
#ifndef ADALN_H
#define ADALN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of x, y, dy, dx, scale and shift (the `dtype` argument). */
typedef enum adaln_dtype { ADALN_F32 = 0, ADALN_BF16 = 1 } adaln_dtype_t;

/* Return codes.  Each has a short alias (ADALN_EINVAL, ...). */
#define ADALN_OK 0
#define ADALN_ERR_INVALID (-1)     /* NULL pointer, bad size or exponent */
#define ADALN_ERR_DTYPE (-2)       /* unknown dtype code */
#define ADALN_ERR_ALIGN (-3)       /* D not a multiple of the vector width,
                                      or a pointer not 16-byte aligned */
#define ADALN_ERR_WORKSPACE (-4)   /* workspace NULL or too small */
#define ADALN_ERR_HIP (-5)         /* the HIP runtime reported an error */
#define ADALN_ERR_UNSUPPORTED (-6) /* D too wide for the entry point */
#define ADALN_EINVAL ADALN_ERR_INVALID
#define ADALN_EDTYPE ADALN_ERR_DTYPE
#define ADALN_EALIGN ADALN_ERR_ALIGN
#define ADALN_EWORKSPACE ADALN_ERR_WORKSPACE
#define ADALN_EHIP ADALN_ERR_HIP
#define ADALN_EUNSUPPORTED ADALN_ERR_UNSUPPORTED

/*
 * Forward pass: mean, rstd and y for every token row, one kernel launch
 * (one per 2^20 workgroups: per 2^22 rows of up to 1024 vectors, 2^21 of up
 * to 1536, 2^20 wider).
 * Section 2.B, forward pass: the row statistics stay in registers (and LDS
 * when several wavefronts share a row) and the modulation is applied on the
 * pass that writes y.
 *   x      [B,N,D] dtype  in
 *   scale  [B,D]   dtype  in
 *   shift  [B,D]   dtype  in
 *   y      [B,N,D] dtype  out
 *   mean   [B,N]   f32    out (saved for the backward pass)
 *   rstd   [B,N]   f32    out (saved for the backward pass)
 * B*N == 0 is a successful no-op.
 */
int adaln_fwd(const void *x, const void *scale, const void *shift, void *y,
              float *mean, float *rstd, int64_t B, int64_t N, int64_t D,
              int dtype, void *stream);

/*
 * Bytes of device workspace the backward entry points (adaln_bwd,
 * adaln_bwd_fused, adaln_bwd_finish, adaln_bwd_dmod) need for this shape:
 * the per-(sample, n_tile) partial sums of the D-tile reduction.
 * A pure function of its arguments.  Returns 0 for invalid arguments.
 */
size_t adaln_bwd_workspace_bytes(int64_t B, int64_t N, int64_t D, int dtype);

/*
 * Backward pass: dx, dscale and dshift.  Section 2.B, backward pass: the
 * gradients of the modulation parameters are sums along the sequence
 * dimension N, taken over a (d_tile, n_tile) grid with every lane pinned to
 * its features so that each access is contiguous along D, then combined
 * across the n_tiles; dx, on which the pages are silent, is the exact
 * gradient of the forward formula above.  It enqueues adaln_bwd_fused then
 * adaln_bwd_finish (x and dy read once) for every row width the library
 * takes; adaln_bwd_dx and adaln_bwd_dmod below are the same gradients as
 * two separate passes.
 *   dy        [B,N,D] dtype in   upstream gradient dL/dy
 *   x         [B,N,D] dtype in   the forward input
 *   scale     [B,D]   dtype in
 *   mean,rstd [B,N]   f32   in   as written by adaln_fwd for this x
 *   dx        [B,N,D] dtype out
 *   dscale    [B,D]   f32   out  (overwritten, not accumulated)
 *   dshift    [B,D]   f32   out  (overwritten, not accumulated)
 *   workspace, workspace_bytes: at least adaln_bwd_workspace_bytes(...)
 *     bytes of device memory; contents on entry are ignored.
 * With B*N == 0 and B*D > 0, dscale and dshift are set to zero.
 */
int adaln_bwd(const void *dy, const void *x, const void *scale,
              const float *mean, const float *rstd, void *dx, float *dscale,
              float *dshift, void *workspace, size_t workspace_bytes,
              int64_t B, int64_t N, int64_t D, int dtype, void *stream);

/*
 * adaln_bwd for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, kernels and results as adaln_bwd
 * (bit for bit), without the workspace: the partial rows go to a static
 * device array of the library, 64 MiB per GPU, held until the process ends.
 * Shapes whose adaln_bwd_workspace_bytes exceeds 64 MiB return
 * ADALN_ERR_WORKSPACE before any HIP call.  The first call on a device looks
 * up the array's device address (hipGetSymbolAddress) and keeps it; make one
 * call before capturing a graph.  Every call on a GPU shares that GPU's
 * array, so calls that overlap on one GPU (other streams, other threads)
 * race and must be ordered by the caller.  Nothing needs clearing between
 * calls: each call writes every partial row it reads.
 */
int adaln_bwd_noalloc(const void *dy, const void *x, const void *scale,
                      const float *mean, const float *rstd, void *dx,
                      float *dscale, float *dshift, int64_t B, int64_t N,
                      int64_t D, int dtype, void *stream);

/*
 * The two launches adaln_bwd makes, exposed so callers can schedule or time
 * them separately.  Rows of up to 320 vectors are owned by one wavefront
 * each, wider ones by a pair of wavefronts (up to 1280 vectors), four (up to
 * 2560) or eight (up to 4096, the widest row; 512-thread workgroups), which
 * combine their row sums through LDS.  adaln_bwd_fused reads x and dy once:
 * it writes dx and, per
 * (sample, n_tile), float32 partial sums of dscale and dshift into the
 * workspace -- the D-tile coalesced reduction of section 2.B with dx fused
 * into the same pass over the rows: one partial row per (sample, workgroup).
 * adaln_bwd_finish then sums those partials over the workgroups of each
 * sample in index order into dscale and dshift.  The
 * workspace must be the one adaln_bwd_fused filled for the same B, N, D and
 * dtype, with no other call using it in between.
 */
int adaln_bwd_fused(const void *dy, const void *x, const void *scale,
                    const float *mean, const float *rstd, void *dx,
                    void *workspace, size_t workspace_bytes, int64_t B,
                    int64_t N, int64_t D, int dtype, void *stream);

int adaln_bwd_finish(const void *workspace, size_t workspace_bytes,
                     float *dscale, float *dshift, int64_t B, int64_t N,
                     int64_t D, int dtype, void *stream);

/*
 * Launch plan of adaln_bwd_fused for this shape, for callers that account
 * for the partial sums it writes: fills out[0..3] with {vectors per lane,
 * wavefronts per row (1, 2, 4 or 8), workgroups launched, partial rows per
 * sample P}.
 * The partials occupy 2*B*P*D floats at the start of the workspace.
 * Host-only; no HIP call.
 */
int adaln_bwd_fused_plan(int64_t B, int64_t N, int64_t D, int dtype,
                         int64_t *out);

/*
 * How adaln_fwd (which = 0) or adaln_bwd_fused (which = 1) splits a batch
 * into work, for callers that account for it and for tests of the planner.
 * Fills out[0..6] with {vectors per lane V, wavefronts per row W, workgroups
 * launched, workgroups per sample bps, samples in flight groups, row walkers
 * per workgroup, skew}.  Workgroup g with g / bps < groups works on samples
 * g / bps, g / bps + groups, ... in turn; in each sample b, its walker w
 * visits the walk positions (g % bps) * walkers + w, then every
 * bps * walkers positions; position n stands for row (n + b * skew) mod N of
 * the sample (skew is 0 except in the backward of many samples).  The
 * backward of bf16 rows of exactly D = 3072 or 5120 (pairs of wavefronts,
 * 3 or 5 vectors per lane) walks in rounds instead: m regular steps as
 * above (m = 12 for D = 3072, 16 for D = 5120), then one extra step for the
 * walkers of workgroups with an even g, which take, in the order of
 * ((g % bps) * walkers + w), the positions that follow the round's regular
 * ones; a round covers m * bps * walkers positions plus one per such
 * walker of the sample.  A walker
 * is one wavefront (W = 1) or the W wavefronts that share a row (a
 * workgroup holds 4 / W walkers, or one when W = 8).  The forward has
 * bps = groups = 0 and covers the B * N rows of the batch with its grid
 * instead: walker j of workgroup g takes row (4 / W) * g + j, in launches
 * of at most 2^20 workgroups; out[2] counts the workgroups of all of them.
 * Host-only; no HIP call.
 *
 * which = 2: the launch that sums the partial rows into dscale and dshift
 * (adaln_bwd_finish).
 * Fills out[0..5] with {features per column block F (16, 32 or 64),
 * wavefronts per block wpc, blocks per workgroup cpb, workgroups launched G,
 * threads per workgroup, partial rows P summed per output}.  Block k covers
 * sample k / C, features (k % C) * F + [0, F), C = ceil(D / F).  Workgroup g
 * takes the blocks L * cpb + [0, cpb), then those of L + G, L + 2G, ...,
 * where L = g, except for F < 64 and g < 8 * (G / 8): L = (g % 8) * (G / 8)
 * + g / 8.  The j-th wpc wavefronts of a workgroup serve its j-th block;
 * wavefront s of them sums the rows [s * P / wpc, (s + 1) * P / wpc).
 * out[6] is 0.
 *
 * which = 3: the (d_tile, n_tile, b) grid of adaln_bwd_dmod's first launch.
 * Fills out[0..6] with {d_tiles (64 vectors of features each), rows per
 * n_tile, n_tiles per sample, workgroups d_tiles * n_tiles * B, threads per
 * workgroup, 0, 0}; its partial sums occupy 2 * B * n_tiles * D floats of
 * the workspace, which the second launch sums over the n_tiles.
 */
int adaln_plan(int which, int64_t B, int64_t N, int64_t D, int dtype,
               int64_t *out);

/*
 * Backward, input gradient only: dx from dy, x, scale and the saved
 * mean/rstd, one kernel launch (arguments as in adaln_bwd).  The pages give
 * no design for dx; it is the exact gradient of the formula above.
 */
int adaln_bwd_dx(const void *dy, const void *x, const void *scale,
                 const float *mean, const float *rstd, void *dx, int64_t B,
                 int64_t N, int64_t D, int dtype, void *stream);

/*
 * Backward, modulation gradients only: dscale and dshift through the D-tile
 * coalesced reduction of section 2.B (backward pass).  Two launches: a
 * (d_tile, n_tile, b) grid in which each lane owns 16 bytes of features and
 * accumulates down the rows of its n_tile in float32, writing per-tile
 * partial sums to the workspace; then a fixed-order sum over the n_tiles.
 * No floating-point atomics: results are bitwise reproducible.
 * Arguments as in adaln_bwd.
 */
int adaln_bwd_dmod(const void *dy, const void *x, const float *mean,
                   const float *rstd, float *dscale, float *dshift,
                   void *workspace, size_t workspace_bytes, int64_t B,
                   int64_t N, int64_t D, int dtype, void *stream);

/*
 * Packed variable-length AdaLN: the token rows of several sequences
 * ("segments") concatenated in one [T, D] tensor and processed in one launch
 * per pass (the forward: one per 2^20 workgroups, as in adaln_fwd)
 * -- mixed-length samples of a bucket without padding, or the text
 * and video token segments of MMDiT samples, each with its own modulation.
 *   seg_offsets  host int64 [nseg+1]: segment s is rows [off[s], off[s+1]);
 *                off[0] = 0, non-decreasing, T = off[nseg] < 2^31
 *   seg_mod      host int32 [nseg] or NULL: segment s is modulated by
 *                scale[seg_mod[s]], shift[seg_mod[s]] (NULL: vector s)
 *   nseg         0 .. 128 segments;  nmod: number of modulation vectors
 *   x, y, dy, dx [T, D] dtype;  mean, rstd [T] f32
 *   scale, shift [nmod, D] dtype;  dscale, dshift [nmod, D] f32, where
 *                dscale[m] sums dy*xhat over every row of every segment
 *                with seg_mod[s] == m (zero for an unused m)
 * The per-row math is that of adaln_fwd / adaln_bwd.  The forward takes every
 * row width adaln_fwd takes, and so does the backward.  The workspace of
 * adaln_bwd_segments is
 * adaln_bwd_segments_workspace_bytes(seg_offsets, nseg, D, dtype) bytes; the
 * host arrays are read during the call only.
 */
int adaln_fwd_segments(const void *x, const void *scale, const void *shift,
                       void *y, float *mean, float *rstd,
                       const int64_t *seg_offsets, const int32_t *seg_mod,
                       int64_t nseg, int64_t nmod, int64_t D, int dtype,
                       void *stream);

size_t adaln_bwd_segments_workspace_bytes(const int64_t *seg_offsets,
                                          int64_t nseg, int64_t D, int dtype);

int adaln_bwd_segments(const void *dy, const void *x, const void *scale,
                       const float *mean, const float *rstd, void *dx,
                       float *dscale, float *dshift, void *workspace,
                       size_t workspace_bytes, const int64_t *seg_offsets,
                       const int32_t *seg_mod, int64_t nseg, int64_t nmod,
                       int64_t D, int dtype, void *stream);

/*
 * Dual-constraint bucket batch size of section 2.A:
 *     max(1, min(floor(m_mem / S), floor(m_comp / S^p)))
 * in exact integer arithmetic.  When S^p exceeds the int64 range the compute
 * bound is 0 and the result is 1.  Returns ADALN_ERR_INVALID for S <= 0,
 * negative bounds or a negative exponent.  Host-only; no HIP call.
 */
int64_t adaln_bshape(int64_t S, int64_t m_mem, int64_t m_comp, int32_t p);

/*
 * The same rule with a fitted, real exponent and compute bound (section 2.A,
 * cost-fitting system): max(1, min(floor(m_mem / S), floor(m_comp / S^p))),
 * the compute bound taken as floor of the double quotient m_comp / pow(S, p).
 * Returns ADALN_ERR_INVALID for S <= 0, a negative or non-finite bound or
 * exponent.  Host-only.
 */
int64_t adaln_bshape_real(int64_t S, int64_t m_mem, double m_comp, double p);

/*
 * Compute bound implied by a fitted exponent (section 2.A, cost-fitting
 * system; how M_comp follows from the fit is not stated there, so it is read
 * as the B * S^p of the memory-bound bucket of a reference length s_ref,
 * which no bucket's predicted cost a + b * B * S^p then exceeds):
 *     (m_mem / s_ref) * s_ref^p      (integer quotient, then a double)
 * With the pages' own p = 2, M_mem = 131072 and s_ref = 16380 this gives
 * 8 * 16380^2 = 2.146e9, the 2.2e9 they quote to two digits.  Returns -1.0
 * (and records ADALN_ERR_INVALID) for s_ref <= 0, m_mem < 0 or an exponent
 * that is negative or not finite.  Host-only.
 */
double adaln_mcomp(double p, int64_t m_mem, int64_t s_ref);

/*
 * Step-time cost model of section 2.A: fits t ~ a + b * B * S^p to n >= 3
 * measured samples (B[i], S[i], t[i]) (host arrays of double; B, S > 0) by
 * least squares over a, b and p in [p_lo, p_hi].  For each p the best (a, b)
 * is the closed-form linear fit; the residual is then minimised over p by a
 * 400-interval grid scan followed by golden-section search.  Writes
 * out[0..3] = a, b, p, residual sum of squares.  Returns ADALN_OK or
 * ADALN_ERR_INVALID (NULL array, n < 3, a non-positive B or S, a non-finite
 * value, p_lo >= p_hi).  Host-only.
 */
int adaln_costfit(const double *B, const double *S, const double *t,
                  int64_t n, double p_lo, double p_hi, double *out);

/* Largest D the row kernels accept for `dtype` (0 for an unknown dtype). */
int64_t adaln_max_d(int dtype);

/* Static, human-readable name of a return code. */
const char *adaln_strerror(int code);

/* The calling thread's message for its most recent failing call ("" if
 * none); valid until that thread's next call into the library. */
const char *adaln_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ADALN_H */
