/*
 * etpc.h -- streaming edge-conditioned O(3) tensor-product convolution for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is the edge-conditioned equivariant convolution of the Sobek
 * paper ("Sobek: Streaming Equivariant Tensor Product Convolutions", Sec. 2,
 * Eq. 6-13):
 *
 *   z_i = sum_{e=(j->i)} sum_{paths pi} sum_{u,w} w_e,pi[u,w] (x_j,u (x)_CG Y(r_e))_pi
 *   w_e,pi = sum_b phi_b(|r_e|) W_pi[b]                     (radial projection, Eq. 12)
 *   r_e = p_j - p_i   (sender minus receiver, Eq. 8; minimum image in a periodic box)
 *
 * in two connection modes: fully connected "uvw" (Eq. 6) and channelwise "uvu"
 * (Eq. 7).  It is evaluated in the streaming order of Sec. 3-4 (Eq. 15-17,
 * 32-36): per-edge weights, messages and weight adjoints are never stored.
 *
 * Conventions (the paper leaves them open; these are this library's readings):
 *  - harmonics: real, component-normalized (sum_m Y_lm^2 = 2l+1), m = -l..l,
 *    l = 1 ordered (y, z, x); degree l has parity (-1)^l; l <= 3.
 *  - coupling c^pi[m_in][m_sh][m_out]: real-basis SO(3) intertwiner, each output
 *    column of unit norm, first nonzero entry (C order) positive; no extra path
 *    normalization factor.
 *  - radial: Gaussian  phi_b = exp(-(r-mu_b)^2/(2D^2)), mu_b = r_lo + b D,
 *    D = (r_hi-r_lo)/(B-1);  Bessel  phi_b = sqrt(2/r_c) sin(b pi r/r_c)/r f_p(r/r_c),
 *    b = 1..B, r_c = r_hi, polynomial envelope f_p of degree p+2 (zero beyond r_c).
 *  - layouts, all row-major fp32 with int32 graph indices:
 *      x, x_bar, x_grad, x_dot : [N][x_dim]   ir_mul: block k stored [2l+1][C], channel fastest
 *      z, z_bar, z_bar_grad    : [N][z_dim]   ir_mul
 *      pos, pos_bar, pos_dot   : [N][3]
 *      w, w_bar, w_grad, w_dot : paths in plan order (out_block, in_block, l_sh),
 *                                uvw block [B][C_in][C_out], uvu block [B][C_in].
 *
 * Ownership: the caller allocates every data and workspace buffer; the library
 * allocates nothing in a compute call.  A plan is host memory only (its tables
 * travel to the GPU as kernel arguments) and is immutable after creation, so it
 * may be shared across streams; concurrent calls need distinct workspaces.
 * Inputs are read-only; outputs are overwritten (never accumulated into).
 * Every call validates its arguments on the host first; on a non-OK status no
 * kernel has been enqueued and etpc_last_error() describes the problem.
 * Compute calls are asynchronous on the given stream; results are
 * deterministic for a given workspace size and plan (fixed reduction owners and orders,
 * no floating-point atomics; timing never changes a result).  Inside a call, the
 * independent per-path launches of a pass run on up to two side streams (etpc_spec.lanes), and the node-side GEMMs of a pass on a third
 * ("post") stream that overlaps them with the next group's or block's traversals; the
 * library creates these streams once per device (default priority) and forks them from
 * and joins them back into the given stream with events, so the call still behaves as
 * one ordered unit of that stream (and can be captured into a HIP graph).  Calls from
 * several host threads serialize their fork-to-join sections on per-device locks; the
 * first call on a device creates the side streams.
 */
#ifndef ETPC_H
#define ETPC_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct etpc_plan_s* etpc_plan;

typedef enum {
  ETPC_OK = 0,
  ETPC_ERR_INVALID_ARG = 1,   /* null required pointer, bad size, bad enum */
  ETPC_ERR_UNSUPPORTED = 2,   /* l > 3, B > 16, more than 64 paths, ... */
  ETPC_ERR_INVALID_PATH = 3,  /* instruction violates the selection rule (Eq. 5) or uvu C_out != C_in */
  ETPC_ERR_WORKSPACE = 4,     /* workspace below the minimum of a pass (one node's state plus its
                                 fixed parts; backward adds 12 B per edge per lane); smaller than
                                 etpc_workspace_size() but above that minimum runs in node chunks */
  ETPC_ERR_OVERFLOW = 5,      /* N, E or an internal index would exceed int32 */
  ETPC_ERR_GRAPH = 6,         /* etpc_graph_validate found an inconsistent CSR */
  ETPC_ERR_HIP = 7,           /* a HIP runtime call failed */
  ETPC_ERR_CAPACITY = 8       /* an output buffer is smaller than the result (the needed size is
                                 returned where the call says) */
} etpc_status;

typedef enum { ETPC_UVW = 0, ETPC_UVU = 1 } etpc_mode;
typedef enum { ETPC_RADIAL_GAUSSIAN = 0, ETPC_RADIAL_BESSEL_POLY = 1 } etpc_radial;
typedef enum { ETPC_PASS_FWD = 0, ETPC_PASS_BWD = 1, ETPC_PASS_DBL = 2 } etpc_pass;
/* Arithmetic of the channel-space GEMMs (z = S W, Xt = x W, x_bar = P W^T, W_bar = x^T P).
 * FP32 is the reference schedule.  BF16 rounds both operands to bf16 (nearest, ties to
 * even) and accumulates in fp32 on the matrix cores: the analogue of the optional TF32
 * channel GEMMs of Sec. 4, with about 2^-9 relative rounding per operand.  FP16 does the
 * same in fp16 (2^-11 relative rounding; magnitudes above 65504 overflow to infinity).
 * The traversals and every reduction stay fp32. */
typedef enum { ETPC_GEMM_FP32 = 0, ETPC_GEMM_BF16 = 1, ETPC_GEMM_FP16 = 2 } etpc_gemm_precision;

/* One irrep block: multiplicity, degree l (0..3) and parity (+1 'e', -1 'o'). */
typedef struct { int32_t mul, l, parity; } etpc_irrep;
/* One instruction (path): input block, harmonic degree, output block. */
typedef struct { int32_t in_block, l_sh, out_block; } etpc_instr;

typedef struct {
  int32_t n_in;  const etpc_irrep* in;        /* [host] input irreps (Eq. 3) */
  int32_t n_out; const etpc_irrep* out;       /* [host] output irreps, or allowed outputs (see below) */
  int32_t out_per_path;  /* uvu only: nonzero = one output block per valid (in, l_sh, allowed out)
                            in that nested order, multiplicity tied to the input (Eq. 7);
                            `out` then lists the allowed (l, parity), `mul` ignored */
  int32_t lmax_sh;                            /* 0..3 */
  int32_t mode;                               /* etpc_mode */
  int32_t n_instr; const etpc_instr* instr;   /* [host] NULL/0 = every valid (in, l_sh, out) */
  int32_t radial;                             /* etpc_radial */
  int32_t n_basis;                            /* B: 1..16 (Gaussian needs >= 2) */
  float r_lo, r_hi;                           /* Gaussian range; Bessel cutoff = r_hi */
  int32_t poly_p;                             /* Bessel envelope exponent p >= 1 */
  float box[3];                               /* all zero = open; else orthorhombic minimum image */
  int32_t gemm_precision;                     /* etpc_gemm_precision; 0 (default) = fp32 */
  int32_t lanes;     /* concurrent launch lanes of a pass: 0 = default (2), 1 = every launch in
                        order on the caller's stream (e.g. to time kernels one at a time), 2 =
                        independent per-path launches on two library side streams plus the
                        node-side GEMMs on a third.  Results do not depend on it beyond the
                        summation order of the per-lane position-adjoint copies (pos_bar). */
} etpc_spec;

/* Receiver-sorted CSR plus the sender (source) view; all DEVICE pointers.
 * rowptr[N+1], col[E] = sender of each receiver slot;
 * s_rowptr[N+1], s_col[E] = receiver of each sender slot, s_slot[E] = the receiver slot.
 * s_order[N] (optional, NULL = index order): the senders by decreasing out-degree within
 * aligned windows of ETPC_SEND_ORDER_WINDOW senders, ties in index order
 * (etpc_degree_order(s_rowptr, ETPC_SEND_ORDER_WINDOW)) or windows and ties taken along a
 * base sequence such as the spatial order (etpc_degree_order_within(s_rowptr,
 * ETPC_SEND_ORDER_WINDOW, etpc_spatial_order(pos))).  r_order[N] (optional): likewise the
 * receivers by in-degree within windows of ETPC_RECV_ORDER_WINDOW.  The uvw traversals then
 * start the longest rows first, which shortens the tail of each launch.  The orders stay
 * window-local so that nodes that are close (numbered together, as the cells of a batch or
 * a space-filling-curve numbering, or consecutive in a spatial base order) still run close
 * together in time and share cache; the sender window is about the number of waves resident
 * on the chip at once, the receiver window a fraction of one XCD's share (the receiver
 * traversals also give each XCD a contiguous range of node slots).  Results are
 * bit-identical for any order.
 * Preconditions (checked only by etpc_graph_validate): indices in range, both views
 * describe the same edge multiset, no self loops, |r_e| > 0 on every edge, s_order and
 * r_order (when given) permutations of the nodes whose degrees do not increase within each
 * aligned window of positions. */
enum { ETPC_SEND_ORDER_WINDOW = 4096, ETPC_RECV_ORDER_WINDOW = 512 };
typedef struct {
  int32_t n_nodes;
  int64_t n_edges;
  const int32_t* rowptr;
  const int32_t* col;
  const int32_t* s_rowptr;
  const int32_t* s_col;
  const int32_t* s_slot;
  const int32_t* s_order;
  const int32_t* r_order;
} etpc_graph;

/* Planner (host only).  Parses the spec, enumerates the valid paths (selection
 * rule, Eq. 5), builds the real coupling tensors in float64 (Racah's formula moved
 * to the real basis) and the block offsets.  Sec. 4, the paragraph on the kernel
 * generator: it enumerates valid paths and sparse CG terms from the irreps. */
etpc_status etpc_plan_create(const etpc_spec* spec, etpc_plan* out);
void etpc_plan_destroy(etpc_plan plan);
/* Widths: x_dim = sum C(2l+1) (Eq. 4), z_dim likewise, w_numel = B * sum n_pi (Eq. 9-10). */
etpc_status etpc_plan_info(etpc_plan plan, int64_t* x_dim, int64_t* z_dim, int64_t* w_numel,
                           int32_t* n_paths);
/* [host] Path p (0 <= p < n_paths) in plan order: one instruction (in_block, l_sh, out_block)
 * that passes the selection rule (Eq. 5), its degrees l_in, l_out, and where its operands
 * live (Eq. 9-10: each path owns one radial-weight block W_pi[b]):
 *   x_off  offset (floats) of the input block within an x row ([2l_in+1][C_in], ir_mul);
 *   z_off  offset (floats) of the output block within a z row ([2l_out+1][C_out]);
 *   w_off, w_numel  the path's block of w: uvw [B][C_in][C_out], uvu [B][C_in];
 *   fan_in = B * (sum of C_in over the paths of the output block) for uvw (the D_g of the
 *            channel GEMM, Eq. 34), B for uvu.
 * Every output pointer may be NULL.  ETPC_ERR_INVALID_ARG for a null plan or p out of range. */
etpc_status etpc_plan_path(etpc_plan plan, int32_t p, int32_t* in_block, int32_t* l_sh, int32_t* out_block,
                           int32_t* l_in, int32_t* l_out, int64_t* x_off, int64_t* z_off, int64_t* w_off,
                           int64_t* w_numel, int32_t* fan_in);
/* Output block b (useful when out_per_path built the output list). */
etpc_status etpc_plan_out_irrep(etpc_plan plan, int32_t b, int32_t* n_out, etpc_irrep* irrep);
/* [host] dense coupling tensor of path p, [2l_in+1][2l_sh+1][2l_out+1] doubles (Eq. 32). */
etpc_status etpc_plan_cg(etpc_plan plan, int32_t p, double* out);

/* [host] Workspace bytes of a compute pass (etpc_pass) over a graph of n_nodes / n_edges.
 * Sec. 4 keeps the tensor-product scratch within a fixed budget (Sec. 5: 128 MiB) by
 * running bounded receiver ranges; here the node-side states (the uvw receiver state S of
 * Eq. 33, the sender state P and Xt of the backward, two sets of each so the GEMMs of one
 * output group or input block overlap the traversals of the next) are sized by a node
 * chunk:
 *   budget == 0: every node in one chunk, the fastest schedule;
 *   budget  > 0: the largest node chunk whose workspace fits in `budget` bytes (the full
 *                size when that already fits).
 * Backward and double backward add 12 B per edge per concurrent lane of the plan (the
 * per-edge position adjoint, in receiver-slot order); nothing scales with E times a
 * channel width.  A compute call given any workspace of at least this many bytes runs
 * with a chunk at least this large; results differ between chunk sizes only in summation
 * order.  ETPC_ERR_WORKSPACE (with *bytes set to the minimum, one node per chunk) when the
 * budget is below that minimum; ETPC_ERR_INVALID_ARG for a null plan or output, negative
 * sizes or an unknown pass. */
etpc_status etpc_workspace_size(etpc_plan plan, int32_t pass, int32_t n_nodes, int64_t n_edges,
                                size_t budget, size_t* bytes);

/* Build both CSR views from a COO list (src[e] -> dst[e]), stable: receiver view sorted
 * by receiver with ties in COO order; sender view sorted by sender with ties in
 * receiver-slot order (Sec. 4: cached stable CSR views give receiver and source
 * reductions fixed ownership).  eid[slot] = COO index.  All arrays are device int32.
 * Bit-exact and deterministic.  Workspace from etpc_csr_workspace_size. */
etpc_status etpc_csr_workspace_size(int32_t n_nodes, int64_t n_edges, size_t* bytes);
etpc_status etpc_csr_build(int32_t n_nodes, int64_t n_edges, const int32_t* src, const int32_t* dst,
                           int32_t* rowptr, int32_t* col, int32_t* eid,
                           int32_t* s_rowptr, int32_t* s_col, int32_t* s_slot,
                           void* ws, size_t ws_bytes, hipStream_t stream);
/* Node dispatch order.  window = 0: order[k] = the node with the k-th largest row
 * length rowptr[v+1] - rowptr[v], ties in increasing node index (a stable sort by
 * decreasing degree).  window > 0: the same within each aligned window of `window`
 * nodes: positions [k w, (k+1) w) hold the nodes [k w, (k+1) w), heaviest first.  The
 * traversals own whole CSR rows (Sec. 4: receiver rows forward, source-contiguous rows
 * backward), so a workgroup's work is its node's degree; starting the heavy nodes first is
 * the longest-first rule of list scheduling.  rowptr [device] int32 [N+1]
 * (non-decreasing); order [device] int32 [N] out.  Bit-exact and deterministic.
 * Workspace from etpc_degree_order_workspace_size; ETPC_ERR_INVALID_ARG for N < 0,
 * window < 0, null pointers with N > 0, or a workspace too small. */
etpc_status etpc_degree_order_workspace_size(int32_t n_nodes, size_t* bytes);
etpc_status etpc_degree_order(int32_t n_nodes, const int32_t* rowptr, int32_t window, int32_t* order, void* ws,
                              size_t ws_bytes, hipStream_t stream);
/* The same along a base sequence: base [device] int32 [N], a permutation of the nodes
 * (e.g. etpc_spatial_order).  window = 0: all nodes by decreasing degree, ties in base
 * order; window > 0: positions [k w, (k+1) w) hold the nodes base[k w .. (k+1) w), heaviest
 * first, ties in base order.  Workspace from etpc_degree_order_workspace_size; the same
 * errors, and ETPC_ERR_INVALID_ARG for a null base (base is not checked to be a
 * permutation). */
etpc_status etpc_degree_order_within(int32_t n_nodes, const int32_t* rowptr, int32_t window, const int32_t* base,
                                     int32_t* order, void* ws, size_t ws_bytes, hipStream_t stream);
/* Spatial node order: the nodes by the Morton (Z-order) code of their position, 10 bits per
 * axis over a 1024^3 grid, ties in increasing node index.  With box [host] float[3]
 * (periodic lengths > 0) each coordinate is wrapped into [0, L) first; with box = NULL the
 * grid spans the points' bounding box.  As the base of the dispatch orders it puts nodes
 * that share neighbours next to each other, so the workgroups that one XCD runs together
 * gather overlapping rows through that XCD's L2 (the traversals' gathers of Sec. 4 read
 * sender rows forward and receiver rows backward).  pos [device] float [N][3]; order
 * [device] int32 [N] out.  Bit-exact and deterministic; no host synchronization.
 * Workspace from etpc_spatial_order_workspace_size; ETPC_ERR_INVALID_ARG for N < 0, null
 * pointers with N > 0, a non-positive or non-finite box length, or a workspace too small. */
etpc_status etpc_spatial_order_workspace_size(int32_t n_nodes, size_t* bytes);
etpc_status etpc_spatial_order(int32_t n_nodes, const float* pos, const float* box, int32_t* order, void* ws,
                               size_t ws_bytes, hipStream_t stream);
/* Debug check of the graph preconditions listed with etpc_graph (Sec. 4: the traversals
 * own whole rows of cached, stable receiver and source CSR views, so both views must
 * describe one edge multiset in the stable orders etpc_csr_build produces; Eq. 8 needs
 * |r_e| > 0).  Checks on the device: rowptr / s_rowptr start at 0, are non-decreasing
 * and end at n_edges; col / s_col in [0, N); no self loops; s_slot a permutation of the
 * receiver slots with s_col[k] = receiver of slot s_slot[k] and col[s_slot[k]] = the
 * sender of row k; each sender row in increasing slot order; s_order / r_order (when
 * given) permutations with non-increasing degree inside each window of positions.
 * Positions are not read, so |r_e| > 0 stays the caller's precondition.  Synchronizes the
 * stream; needs no workspace (it allocates N ints of its own while checking the orders).
 * ETPC_ERR_GRAPH with a description of the first violation found; ETPC_ERR_INVALID_ARG
 * for null arrays or negative sizes. */
etpc_status etpc_graph_validate(const etpc_graph* graph, hipStream_t stream);

/* Graph preparation: the radius graph of N points (the workloads of Sec. 3 are radius
 * graphs, |E| growing as |V| rho r_c^3; the wrapper of Sec. 4 prepares the graph).
 *   pos      [device] float [N][3]; finite.
 *   cutoff   r_c > 0, finite.
 *   box      [host] float[3] orthorhombic box edge lengths, each >= 2 r_c (minimum image,
 *            at most one image within the cutoff), or NULL for open boundaries.
 *   src, dst [device] int32 [max_edges] outputs: one edge j -> i for every ordered pair
 *            (i != j) with 0 < |r|^2 < r_c^2, sorted by receiver, then sender.
 *   n_edges  [host] out: the number of edges (also when it exceeds max_edges).
 * The edge test is taken in float32 with every operation rounded on its own (no fused
 * multiply-add): d_a = p_j,a - p_i,a, periodic d_a -= L_a rint(d_a (1/L_a)),
 * |r|^2 = (d_x^2 + d_y^2) + d_z^2, compared with r_c * r_c; so the edge set depends on
 * the positions only, never on the cell grid used to find it.  Bit-exact and
 * deterministic.  Synchronizes the stream twice (to size the cell grid and to read the
 * edge count), so it cannot be captured into a HIP graph.  Returns ETPC_ERR_CAPACITY,
 * with *n_edges set and the outputs untouched, when max_edges is too small;
 * ETPC_ERR_OVERFLOW for N >= 2^30 or 2^31 edges or more.  Workspace from
 * etpc_radius_graph_workspace_size: about 36 B per node and 16 B per edge of capacity. */
etpc_status etpc_radius_graph_workspace_size(int32_t n_nodes, int64_t max_edges, size_t* bytes);
etpc_status etpc_radius_graph(int32_t n_nodes, const float* pos, float cutoff, const float* box,
                              int64_t max_edges, int32_t* src, int32_t* dst, int64_t* n_edges,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/* Layout adapter (Sec. 4: kernels use ir_mul, the wrapper transposes the common mul_ir
 * layout at the boundary).  Converts N feature rows of the plan's input irreps
 * (features = ETPC_FEATURES_IN: x, x_bar, x_dot) or output irreps (ETPC_FEATURES_OUT: z,
 * z_bar) between mul_ir (block k stored [C][2l+1]) and ir_mul ([2l+1][C]).  in and out
 * are device [N][width] and must not overlap.  Asynchronous, allocates nothing, no
 * workspace; bit-exact (pure data movement). */
typedef enum { ETPC_TO_IR_MUL = 0, ETPC_TO_MUL_IR = 1 } etpc_layout_dir;
typedef enum { ETPC_FEATURES_IN = 0, ETPC_FEATURES_OUT = 1 } etpc_features;
etpc_status etpc_layout_convert(etpc_plan plan, int32_t features, int32_t direction, int32_t n_nodes,
                                const float* in, float* out, hipStream_t stream);

/* Forward: z = conv(x, pos, W) (Eq. 11-13), streaming order Eq. 32-35 (uvw: receiver
 * state S then a channel GEMM; uvu: edge-local weights, Eq. 17). */
etpc_status etpc_forward(etpc_plan plan, const etpc_graph* graph, const float* x, const float* pos,
                         const float* w, float* z, void* ws, size_t ws_bytes, hipStream_t stream);

/* Forward for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same result as etpc_forward
 * (up to the summation order of node chunks), with no workspace argument.  Its scratch is
 * a fixed 128 MiB device array inside the library (one per GPU, held until the process
 * ends); graphs whose receiver state needs more are run in node chunks that fit.  It
 * calls no hipMalloc, hipFree or other allocating routine and runs every launch in order
 * on `stream` (no side streams).  Every call on one GPU shares that GPU's array and
 * leaves its last contents there: calls that overlap in time on one GPU (two streams, or
 * two host threads) race and give undefined results; calls ordered on one stream do not.
 * ETPC_ERR_WORKSPACE when one receiver's state alone exceeds the 128 MiB (a clear message
 * names both sizes); other errors as etpc_forward. */
etpc_status etpc_forward_noalloc(etpc_plan plan, const etpc_graph* graph, const float* x, const float* pos,
                                 const float* w, float* z, hipStream_t stream);

/* Backward: gradients of <z_bar, z> with respect to x, W and positions (Eq. 18-22 and
 * the chain rule through Eq. 8).  Each output pointer may be NULL to skip it. */
etpc_status etpc_backward(etpc_plan plan, const etpc_graph* graph, const float* x, const float* pos,
                          const float* w, const float* z_bar,
                          float* x_bar, float* w_bar, float* pos_bar,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/* Double backward: vector-Jacobian product of backward (x, W, pos, z_bar) -> (x_bar, W_bar,
 * pos_bar) with cotangents (x_dot, w_dot, pos_dot) (directional second adjoints, Eq. 23-31,
 * channel identities Eq. 37-39).  Returns d/dz_bar, d/dx, d/dW and d/dpos ([N][3]); any
 * cotangent may be NULL (= zero) and any output may be NULL (skipped).  d/dpos holds the
 * position Hessian of each edge's term applied to r_dot_e = pos_dot_sender - pos_dot_receiver
 * (second derivatives of the harmonics and the radial basis, owned by the edge as the
 * pages describe for second order), plus the position adjoint of the x_dot and w_dot terms. */
etpc_status etpc_double_backward(etpc_plan plan, const etpc_graph* graph, const float* x,
                                 const float* pos, const float* w, const float* z_bar,
                                 const float* x_dot, const float* w_dot, const float* pos_dot,
                                 float* z_bar_grad, float* x_grad, float* w_grad, float* pos_grad,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/* Kernel timing (off by default), a measurement aid outside the compute path.  While
 * enabled, every kernel the library enqueues is bracketed by a pair of HIP events recorded
 * on its launch stream, grouped by kind.  etpc_profile_read synchronizes on the recorded
 * events and returns the summed durations (milliseconds) and launch count of one kind
 * since the last enable.  Process-wide (a timer of the whole library, as a profiler is);
 * it never changes what a call computes.  Not meant for concurrent use from several
 * threads. */
typedef enum {
  ETPC_KIND_CSR = 0,          /* CSR build kernels */
  ETPC_KIND_FWD_TRAVERSE = 1, /* receiver traversals (uvw state S, uvu outputs) */
  ETPC_KIND_CHANNEL_GEMM = 2, /* m = S W */
  ETPC_KIND_BWD_TRAVERSE = 3, /* sender traversals (P state, edge position adjoint) */
  ETPC_KIND_NODE_GEMM = 4,    /* Xt = x W, x_bar = P W^T, W_bar = x^T P */
  ETPC_KIND_AUX = 5,          /* weight re-layout, fixed-order reductions, fills, pos_bar */
  ETPC_KIND_PREP = 6,         /* radius graph and layout conversion */
  ETPC_KIND_COUNT = 7
} etpc_kind;
etpc_status etpc_profile_enable(int32_t enable);
etpc_status etpc_profile_read(int32_t kind, double* total_ms, int64_t* launches);

/* Thread-local description of the last non-OK status (empty string if none). */
const char* etpc_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* ETPC_H */
