/*
 * nm_sparse.h -- C ABI of the MI355X (gfx950) N:M semi-structured sparse
 * weight x dense activation product
 *
 *     Y[R][T] = epilogue( (mask (.) W)[R][K] . X[K][T] )
 *
 * The operation is the N:M sparse matrix multiply of "Realizable N:M Sparse
 * Transformer Inference via Search-Kernel Co-Design" (arXiv 2607.12505):
 * Sec. 2.1 defines the constraint (N nonzeros kept in every group of M
 * weights), Sec. 4.1 lists the three mechanisms of its kernel (packed weights
 * for light decoding, micro-dense MMA-aligned execution, adaptive
 * parallelism) and Sec. 4.2 the packed representation that stores each
 * window's kept values together with their positions.  This library is a new
 * design of that operation for CDNA4; it computes exactly the same product.
 *
 * Conventions (all matrices row-major, element strides given in elements):
 *   W  [R][K]  weights, row stride ldw >= K
 *   X  [K][T]  activations, tokens contiguous, row stride ldx >= T
 *   Y  [R][T]  output, row stride ldy >= T
 * Groups are M consecutive elements along K starting at k = 0 (K % M == 0).
 *
 * Ownership: the caller allocates and owns every buffer (weights, packed
 * values / meta, X, Y, bias, scale, workspace); device buffers are HIP device
 * memory.  The library never allocates or frees, and keeps no mutable state
 * beyond a per-device cache of the compute-unit count (filled race-free);
 * inputs are not modified; Y is fully overwritten.  `stream` is a hipStream_t
 * (NULL = the default stream); work is enqueued asynchronously on it.
 *
 * Errors: every argument is validated on the host before anything is
 * enqueued; on an error nothing is launched.  A launch failure reported by the
 * HIP runtime returns NM_EHIP.  Faults inside a kernel surface at the
 * caller's next synchronisation.  All functions are thread-safe.
 */
#ifndef NM_SPARSE_H
#define NM_SPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NM_OK = 0,
  NM_EINVAL = 1,        /* bad argument: null pointer, bad size, N/M, stride, buffer size */
  NM_EUNSUPPORTED = 2,  /* valid but not provided: M not in {4, 8}, dtype pair, alignment */
  NM_EHIP = 3           /* the HIP runtime reported an error at launch */
} nm_status;

typedef enum { NM_I8 = 0, NM_F16 = 1, NM_BF16 = 2, NM_I32 = 3, NM_F32 = 4 } nm_dtype;

/* Activation fused into nm_spmm_act's epilogue. */
typedef enum { NM_ACT_NONE = 0, NM_ACT_GELU = 1 } nm_act;

/* Operand layouts: X [K][T] and Y [R][T] (tokens contiguous, as nm_spmm
 * takes them), or the PyTorch-linear layout X [T][K] and Y [T][R] (the
 * reduction and output dimensions contiguous), which nm_spmm_tk takes. */
typedef enum { NM_LAYOUT_KT = 0, NM_LAYOUT_TK = 1 } nm_layout;

#define NM_FORMAT_VERSION 1u

/*
 * Packed weights (the paper's packed window representation, Sec. 4.2, in a
 * layout chosen for gfx950).  Plain data: fill rows, K, N, M, dtype, the two
 * device buffers and their sizes (from nm_pack_size); nm_pack sets
 * format_version.  Layout, with b = element bytes, KB = 128 / b dense columns
 * per block, w = log2(M), C = (KB / M) * N kept slots per block row:
 *   the matrix is cut into blocks of 16 rows x KB columns, numbered
 *   rb * ceil(K / KB) + kb; block n's values start at n * 16 * C * b bytes,
 *   row rr of the block at rr * C * b, slot c at c * b: slot c is kept member
 *   c % N (ascending in-group position) of group kb * (KB / M) + c / N.
 *   meta (absent when N == M): block n at n * 16 * MR bytes, MR = ceil(C*w/8)
 *   rounded up to a multiple of 4; row rr at rr * MR; slot c's in-group
 *   position in bits [c*w, c*w + w) of the row's little-endian bitstream.
 *   Slots outside the R x K matrix hold value 0 and position c % N.
 * One block row is 128 * N / M bytes of values for every dtype, and one block
 * is the A operand of one gfx950 sparse matrix instruction.
 */
typedef struct {
  int64_t rows;             /* R */
  int64_t K;                /* dense reduction length, multiple of M */
  int32_t N, M;             /* N kept of every M */
  int32_t dtype;            /* nm_dtype of the weights: NM_I8, NM_F16 or NM_BF16 */
  uint32_t format_version;  /* NM_FORMAT_VERSION, written by nm_pack */
  void* values;             /* device, values_bytes */
  size_t values_bytes;
  void* meta;               /* device, meta_bytes (may be NULL when N == M) */
  size_t meta_bytes;
} nm_packed;

/*
 * Sizes of the two packed buffers (the packed window representation of
 * Sec. 4.2 -- each window's kept values with their in-window positions -- for
 * the N:M constraint of Sec. 2.1) for an R x K weight of the given N:M and
 * dtype.  NM_EINVAL: null outputs, rows < 1, K < M, K % M != 0, N < 1 or
 * N > M.  NM_EUNSUPPORTED: M not in {4, 8}, dtype not I8 / F16 / BF16.
 * meta_bytes is 0 when N == M.
 */
nm_status nm_pack_size(int64_t rows, int64_t K, int32_t N, int32_t M, int32_t dtype,
                       size_t* values_bytes, size_t* meta_bytes);

/*
 * Select and pack (Sec. 2.1 constraint, Sec. 4.2 packed windows).  For every
 * row and every group of M consecutive K-elements, keep the N members of
 * largest magnitude, equal magnitudes going to the lower position (fp16 /
 * bf16 magnitudes are compared as the sign-cleared bit patterns, which orders
 * every finite value by |w| with +0 == -0, every infinity above every finite
 * value, every NaN above every infinity and NaNs by payload, the sign never
 * mattering), and write them with their positions in the layout above.  W is device memory [rows][ldw] of
 * desc->dtype; desc->values / desc->meta are caller-allocated device buffers
 * of exactly the sizes nm_pack_size returns (NM_EINVAL otherwise).
 * Requires ldw >= K and W 2-byte aligned for 16-bit dtypes.
 */
nm_status nm_pack(const void* W, int64_t ldw, nm_packed* desc, void* stream);

/*
 * Device workspace nm_spmm needs for this weight, token count and output
 * dtype; 0 when none is needed.  It holds the partial sums of a K split
 * across workgroups (the adaptive parallelism of the paper's Sec. 4.1: when
 * the output has too few tiles to occupy the GPU, K is cut into S slices that
 * run as separate work items): S * rows * T * 4 bytes, int32 or fp32, which a
 * second kernel on the same stream adds in slice order before the epilogue.
 * The split is a function of the shape and the device (nm_spmm_ksplit), so
 * the size is too.  For a 1:4, 1:8 or 2:8 int8 weight with a large product
 * (R K T >= 2^31; either operand layout) it instead holds a copy of the weight re-packed
 * into the 2:4 layout (such a pattern is also a 2:4 pattern), which the 2:4
 * sparse-MFMA kernels then multiply: the 2:4 values_bytes rounded up to 256,
 * then the 2:4 meta_bytes.  For another int8 N:M (3:4, 3:8 .. 7:8) with
 * K in (640, 768] and a large product ([K][T] layout) it holds the weight
 * split exactly into two 2:4 layers (every aligned group of four columns
 * keeps at most four members: the first two nonzero ones in the first layer,
 * the rest in the second), each laid out as the re-pack copy above and
 * rounded up to 256 bytes, the second after the first (a dense int8 weight,
 * N = M, needs no copy: the kernel takes the two layers in registers).
 * Given less than that
 * (or a workspace not 256-byte aligned), nm_spmm runs the N:M kernel
 * instead, with the same result.
 * (nm_spmm_tk sizes its workspace with nm_spmm_tk_workspace_size.)
 * The caller owns the buffer; nm_spmm only writes it and
 * reads it back within the call's stream order, so calls that share one
 * workspace must be ordered on one stream.
 */
nm_status nm_spmm_workspace_size(const nm_packed* w, int64_t T, int32_t y_dtype, size_t* bytes);

/*
 * The same for nm_spmm_tk (the [T][K] layout).  Besides the needs above (a
 * 2:4 re-pack for the layout's int8 2:4 kernel), a large call (R K T >=
 * 2^26) whose operands no [T][K] kernel takes runs through the [K][T]
 * kernels: its workspace then holds X transposed to [K][T'] (T' = T rounded
 * up to 16, each part 256-byte aligned), the [K][T'] product before its
 * transpose into Y, and that product's K-split partials if any.  Given less,
 * the call runs the generic kernel instead, with the same result.
 */
nm_status nm_spmm_tk_workspace_size(const nm_packed* w, int64_t T, int32_t y_dtype, size_t* bytes);

/*
 * The N:M sparse product (Sec. 2.1's constrained weight times the
 * activations; Sec. 4.2: only the kept values of each window enter it):
 * Y = epilogue(acc), acc[r][t] = sum over kept slots (r, k) of W[r][k] X[k][t].
 * Supported (weight dtype -> y_dtype) pairs and epilogues:
 *   I8  -> I32 : y = acc + bias[r]                (int32 accumulate, exact)
 *   I8  -> I8  : y = sat_[-128,127](rne(f32(acc + bias[r]) * scale[r]))
 *                (int32 add, RNE conversion, one binary32 multiply, round
 *                half to even, saturate; scale required)
 *   F16 -> F16 / F32,  BF16 -> BF16 / F32 :
 *                y = round_to_y(acc + bias[r]), acc in fp32 (products exact)
 * bias: NULL or device int32[R] (I8 weights) / float[R] (fp weights).
 * scale: device float[R], required iff y_dtype == NM_I8, else ignored.
 * X: device [K][ldx] of the weight dtype; Y: device [R][ldy] of y_dtype.
 * workspace: device, at least nm_spmm_workspace_size bytes, 16-byte aligned
 * (may be NULL if that size is 0).  Under a K split the fp32 sums are added
 * slice by slice, so fp results differ from an unsplit run by rounding only
 * (int32 results are identical).
 * NM_EINVAL: null pointers, T < 1, ldx < T, ldy < T, bad descriptor (sizes
 * not those of nm_pack_size, wrong format_version), small workspace.
 * NM_EUNSUPPORTED: dtype pair not listed, X / Y not aligned to their element,
 * a needed workspace not 16-byte aligned.
 * T is unbounded; R and K are those of the packed weight.
 */
nm_status nm_spmm(const nm_packed* w, const void* X, int64_t ldx, int64_t T, void* Y, int64_t ldy,
                  int32_t y_dtype, const void* bias, const float* scale, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * nm_spmm with an activation fused into the epilogue, for the MLP's first
 * linear layer (the pages' workloads spend their time in the four linear
 * layers of each Transformer block, Sec. 1; the activation between the two
 * MLP layers is not described there -- GELU(x) = x Phi(x) =
 * 0.5 x (1 + erf(x / sqrt 2)), the ViT / Swin activation, is the reading
 * adopted).  Arguments as nm_spmm, plus:
 *   act: NM_ACT_NONE (exactly nm_spmm) or NM_ACT_GELU.
 *   out_scale: with an activation and y_dtype == NM_I8, the requantisation
 *     splits in two around it:
 *       y = sat_[-128,127](rne(act(f32(acc + bias[r]) * scale[r]) * out_scale))
 *     (scale[r] dequantises to the layer's real output, out_scale quantises
 *     the activation's output); ignored otherwise.  Computed in binary32, so
 *     where the exact value lies within a few binary32 ulps of a half-integer
 *     either neighbouring code may result.
 * fp outputs: y = round_to_y(act(acc + bias[r])), act in binary32.
 * NM_EUNSUPPORTED: act not listed, or an activation with y_dtype == NM_I32
 * (raw accumulators); NM_EINVAL: out_scale not finite.
 */
nm_status nm_spmm_act(const nm_packed* w, const void* X, int64_t ldx, int64_t T, void* Y, int64_t ldy,
                      int32_t y_dtype, const void* bias, const float* scale, int32_t act, float out_scale,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * nm_spmm_act in the PyTorch-linear layout: Yt = epilogue(Xt . (mask (.) W)^T)
 * with Xt [T][ldx] (row t holds token t's K activations, K contiguous) and Yt
 * [T][ldy] (row t holds token t's R outputs), so a linear layer's input and
 * output need no transposes.  Same arithmetic, epilogues, activations and
 * errors as nm_spmm_act; ldx >= K and ldy >= R (NM_EINVAL otherwise).
 */
nm_status nm_spmm_tk(const nm_packed* w, const void* Xt, int64_t ldx, int64_t T, void* Yt, int64_t ldy,
                     int32_t y_dtype, const void* bias, const float* scale, int32_t act, float out_scale,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * nm_spmm_act without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  It allocates nothing: the workspace nm_spmm_act
 * would take (K-split partial sums, a 2:4 re-pack of a 1:4 / 1:8 / 2:8 int8
 * weight, the two-layer split of another int8 N:M) is a scratch array of nm_spmm_noalloc_max_bytes() = 32 MiB that the
 * library holds on each device it runs on until the process ends.  Same
 * arguments, arithmetic and results as nm_spmm_act ([K][T] layout).  A call
 * whose K split needs more partial-sum bytes than the scratch holds returns
 * NM_EINVAL before launching anything; a re-pack or split copy that does not fit makes
 * the call run the N:M kernel instead (same result).  No kernel relies on
 * what an earlier call left in the scratch.  Every call on one device shares
 * its scratch: calls that overlap on one device (different streams, threads
 * without ordering) race and must be ordered by the caller.  NM_EHIP: the
 * scratch's device address could not be obtained.
 */
nm_status nm_spmm_noalloc(const nm_packed* w, const void* X, int64_t ldx, int64_t T, void* Y, int64_t ldy,
                          int32_t y_dtype, const void* bias, const float* scale, int32_t act, float out_scale,
                          void* stream);

/* Bytes of the scratch nm_spmm_noalloc uses (its maximum workspace). */
size_t nm_spmm_noalloc_max_bytes(void);

/* Static description of a status code (never NULL). */
const char* nm_status_str(nm_status s);

/*
 * Name of the kernel variant nm_spmm would launch for these arguments
 * (static string; "invalid" when the arguments would be rejected).  A 1:4,
 * 1:8 or 2:8 product re-packed to 2:4 in the workspace is named
 * "repack24_" + the 2:4 kernel's name, the two-layer split
 * "split24_smfmac_i8_stationary" (a dense int8 weight taken as two layers
 * in registers: "dense24_smfmac_i8_stationary"), a [T][K] call run through the [K][T]
 * kernels "transpose_" + that kernel's name (assuming the workspace
 * nm_spmm_workspace_size asks for).  For tests and profiling; launches
 * nothing.
 */
const char* nm_spmm_variant(const nm_packed* w, int64_t T, int32_t y_dtype);

/* The same for nm_spmm_act with activation `act` (which kernels carry it
 * can change the choice). */
const char* nm_spmm_variant_act(const nm_packed* w, int64_t T, int32_t y_dtype, int32_t act);

/* The same for nm_spmm_tk (dense rows: ldx = K, ldy = R). */
const char* nm_spmm_variant_tk(const nm_packed* w, int64_t T, int32_t y_dtype, int32_t act);

/*
 * Number of K slices nm_spmm_act (nm_spmm: act = NM_ACT_NONE) would split
 * this call into across workgroups (1: no split; 0 when the arguments would
 * be rejected), for dense row-major X and Y as nm_spmm_variant assumes.
 * NM_SPMM_VARIANT=<variant>:<S> in the environment (or ":<S>" with the
 * automatic variant) forces S slices where S divides the column blocks and
 * the variant takes a split (1 turns the split off).  Launches nothing.
 */
int32_t nm_spmm_ksplit(const nm_packed* w, int64_t T, int32_t y_dtype, int32_t act);

/* ------------------------------------------------------------------------
 * Three-layer format for moderately unstructured fp16 / bf16 weights (page
 * "Accelerating GPU Inference of Large Language Models with Moderately
 * Unstructured Sparse Weight Matrices", Methodology 1 and 2): any sparse
 * weight is stored exactly as
 *   1. a Sparse-TC layer: the 2:4 packed layout above (N = 2, M = 4) holding
 *      the two largest nonzeros of every group of four (the nm_pack order),
 *      2-bit positions;
 *   2. a Slot-Filling layer: the other nonzeros of groups with three or four
 *      ("surplus") moved into the Sparse-TC layer's empty slots, their
 *      columns given by 4-bit relative distances (PDD), with dummy points
 *      breaking gaps longer than 15;
 *   3. a Residual layer in CSR: surplus that found no slot or code.
 * Geometry: nRB = ceil(rows / 16), nKB = ceil(K / 64), nSeg = ceil(nKB / 8);
 * segment s = column blocks 8s .. 8s+7 (512 columns).  Slot filling works
 * inside a fill unit (row r, segment s, quad q = 0..3): in every block of
 * the segment the 16 columns 64 kb + 16 q .. + 15, which is what one lane
 * holds of the sparse matrix instruction's A operand.  Unit column
 * u = 16 (kb - 8 s) + column % 16, unit slot sigma = 8 (kb - 8 s) + 2 t + j
 * (group t = 0..3 of the quad, slot j).
 *   values / meta: the 2:4 layout; a group with one nonzero at p stores it in
 *     slot 0 at position p and marks slot 1 empty with position p; a group
 *     with none marks both slots empty with positions 1 and 0 (position
 *     pairs never produced by a group with two nonzeros, which are
 *     ascending).  Empty slots hold a slot-filled value or +0.
 *   codes: 8 bytes per unit at ((rb * nSeg + s) * 64 + 16 q + rr) * 8, sixteen
 *     4-bit codes (code i in bits 4 (i % 2) of byte i / 2).  Read in order
 *     from position -1: code 0 is a dummy point (advance 15, no value), code
 *     d in 1..15 advances d to the next surplus element, whose value is in
 *     the unit's next empty slot (ascending sigma).  The packer takes the
 *     unit's surplus in ascending column, greedily, while slots and codes last.
 *   res_ptr / res_ent: CSR over segment rows z = (rb * nSeg + s) * 16 + rr:
 *     nRB * nSeg * 16 + 1 int32 pointers, entries (column - 512 s) << 16 |
 *     value bits (uint32), ascending column within a segment row.
 * ---------------------------------------------------------------------- */
typedef struct {
  int64_t rows, K;          /* R, K (K % 4 == 0) */
  int32_t dtype;            /* NM_F16 or NM_BF16 */
  uint32_t format_version;  /* NM_FORMAT_VERSION, written by nm_hybrid_pack */
  void* values;  size_t values_bytes;   /* Sparse-TC values */
  void* meta;    size_t meta_bytes;     /* Sparse-TC positions */
  void* codes;   size_t codes_bytes;    /* Slot-Filling PDD codes */
  void* res_ptr; size_t res_ptr_bytes;  /* Residual CSR row pointers (int32) */
  void* res_ent; size_t res_ent_bytes;  /* Residual CSR entries (uint32; may be NULL when n_res == 0) */
  int64_t n_fill;           /* slot-filled elements */
  int64_t n_res;            /* residual elements */
} nm_hybrid;

/*
 * Fill desc's rows, K, dtype, the five byte sizes, n_fill and n_res for the
 * weight W (host memory, [rows][ldw] of dtype).  The pointers are left
 * alone.  NM_EINVAL: null W / desc, rows < 1, K < 4, K % 4 != 0, ldw < K, or
 * more than 2^31 - 1 residual entries.  NM_EUNSUPPORTED: dtype not F16 / BF16.
 */
nm_status nm_hybrid_pack_size(const void* W, int64_t ldw, int64_t rows, int64_t K, int32_t dtype,
                              nm_hybrid* desc);

/*
 * Write the three-layer image of W (host memory, as above) into the five
 * HOST buffers desc points to, which the caller allocates with the sizes
 * nm_hybrid_pack_size wrote (res_ent may be NULL when n_res is 0); copying
 * them to device memory is the caller's.  Offline, once per weight; runs on
 * the calling thread plus worker threads it joins before returning.
 * NM_EINVAL as for nm_hybrid_pack_size, for a null buffer, or when desc's
 * sizes or shape do not match W.
 */
nm_status nm_hybrid_pack(const void* W, int64_t ldw, nm_hybrid* desc);

/*
 * Y = epilogue(W X) for a weight in the three-layer format (Methodology 2 of
 * the page: the Slot-Filling codes are decoded by the vector units, the
 * Sparse-TC layer and the decoded slot-filled elements run on the sparse
 * matrix instruction, the residual is accumulated by the vector units in a
 * separate buffer added at the end; loads of the next unit overlap the
 * decode of the current one).  desc's five buffers are device memory.  X is
 * [K][ldx] of the weight's dtype, Y [rows][ldy] of y_dtype (the weight's
 * dtype or NM_F32); bias NULL or float[rows]; act NM_ACT_NONE or
 * NM_ACT_GELU.  Asynchronous on `stream`; allocates nothing.  NM_EINVAL: null
 * pointers, T < 1, ldx < T, ldy < T, a descriptor whose sizes do not match
 * its shape; NM_EUNSUPPORTED: other dtypes, X / Y / buffers not 16-byte
 * aligned, T > 16 tokens per call with K > 4096 (tiles of 16 tokens repeat
 * the decode), version mismatch; NM_EHIP: launch failure.
 */
nm_status nm_hybrid_spmm(const nm_hybrid* w, const void* X, int64_t ldx, int64_t T, void* Y, int64_t ldy,
                         int32_t y_dtype, const void* bias, int32_t act, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NM_SPARSE_H */
