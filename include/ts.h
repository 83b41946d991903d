/*
 * ts.h -- C ABI of the MI355X (gfx950) sparse-convolution library.
 *
 * The library computes sparse convolution over coordinate/feature sparse
 * tensors as the torch-lattice page "Migrating from TorchSparse" states the
 * problem (section "Sparse tensor expectations"): coordinates are int32 rows
 * (batch, x, y, z) -- or (batch, x, y) in 2-D -- with the batch id inside
 * each row, and feature row i of a dense (N, C) matrix belongs to coordinate
 * row i.  Section "Convolution mapping" fixes the support rules: a
 * submanifold convolution keeps the input coordinate set, a strided
 * convolution creates a downsampled one.  Section "Backend and configuration
 * differences" fixes that the dataflow (implicit GEMM, gather-scatter) is a
 * performance choice that must not change the result beyond floating-point
 * rounding, and names the hash-table reserve ratio.
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 * - Memory: the caller allocates every device buffer; the library never
 *   allocates device memory.  Size queries (ts_hash_capacity,
 *   ts_hash_table_bytes, ts_kmap_bytes, ts_conv_workspace_bytes and the
 *   *_scratch_bytes functions) say how much; for arguments the matching call
 *   refuses (negative counts, more than 2^31 - 1 rows or candidates,
 *   unsupported shapes) the byte queries return 0.  All pointers named "device" must be device memory of the current
 *   HIP device; feature matrices are row-major and contiguous.
 * - Streams: every call is asynchronous and ordered on `stream`; there is no
 *   host synchronisation inside the library.  Counts that only the device
 *   knows (the number of strided output rows) are written to device int64
 *   scalars.
 * - Errors: problems visible on the host (null pointers, negative sizes,
 *   unsupported shapes or dtypes, short buffers) return a status before any
 *   launch.  A failed launch returns TS_ERR_HIP.  Problems only the device
 *   sees are ORed into a caller-zeroed uint32 flag word (TS_FLAG_*): the call
 *   still returns TS_OK, and the caller reads the word after synchronising.
 *   Nothing aborts and no exception crosses the ABI.
 * - Coordinates: batch in [0, 65534], spatial values in [-32768, 32767].
 *   A row outside that range is left out of the hash table (it neither finds
 *   nor is found) and raises TS_FLAG_RANGE.  A repeated coordinate keeps its
 *   lowest row and raises TS_FLAG_DUP.
 * - Kernel offsets: offset o of a kernel of size K in D dims is the
 *   displacement delta with delta_d in {-r, ..., K-1-r}, r = (K-1)/2, the
 *   first spatial axis varying slowest:  o = sum_d (delta_d + r) K^(D-1-d).
 *   Weights are [K^D][Cin][Cout]; the convolution is a cross-correlation:
 *     submanifold:  y[j] = sum_o x[row(q_j + delta_o)] . W[o]
 *     strided (s):  y[j] = sum_o x[row(s q_j + delta_o)] . W[o]
 *   with absent rows contributing nothing.  K^D <= 64.
 */
#ifndef TS_H_
#define TS_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The *_RANGE_MIN_ / *_RANGE_MAX_ enumerators are no values of their own:
 * they make every int a value of the enum type, so that an out-of-range
 * value a C caller passes reaches the library's checks (and is refused with
 * TS_ERR_INVALID_ARG) as a defined value. */
typedef enum ts_status {
  TS_OK = 0,
  TS_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad shape, short buffer */
  TS_ERR_UNSUPPORTED = 2, /* valid request this library does not implement      */
  TS_ERR_HIP = 3,         /* a HIP launch or runtime call failed                 */
  TS_STATUS_RANGE_MIN_ = INT32_MIN, TS_STATUS_RANGE_MAX_ = INT32_MAX
} ts_status;

typedef enum ts_dtype {
  TS_F32 = 0, TS_F16 = 1, TS_BF16 = 2,
  TS_DTYPE_RANGE_MIN_ = INT32_MIN, TS_DTYPE_RANGE_MAX_ = INT32_MAX
} ts_dtype;

typedef enum ts_dataflow {
  TS_DATAFLOW_AUTO = 0,          /* per-shape choice                                   */
  TS_DATAFLOW_IMPLICIT_GEMM = 1, /* output-stationary tiles, MFMA for fp16/bf16        */
  TS_DATAFLOW_GATHER_SCATTER = 2, /* per offset: gather, multiply, add into the outputs */
  TS_DATAFLOW_IMPLICIT_GEMM_PACKED = 3, /* implicit GEMM on weights that ts_conv_pack_weights
                                           already wrote into the workspace (w is ignored)  */
  TS_DATAFLOW_FETCH_ON_DEMAND = 4, /* per-tile pair groups: each group of 16 pairs of one offset
                                     fetches its source rows inside the MFMA loop and adds into
                                     an on-chip accumulator tile (maps built with TS_KMAP_GROUPS) */
  TS_DATAFLOW_RANGE_MIN_ = INT32_MIN, TS_DATAFLOW_RANGE_MAX_ = INT32_MAX
} ts_dataflow;

/* device-detected conditions, ORed into the caller's flag word */
#define TS_FLAG_DUP 1u   /* a coordinate appeared twice; its lowest row owns it */
#define TS_FLAG_RANGE 2u /* a coordinate was outside the packable range         */
#define TS_FLAG_FULL 4u  /* the hash table had no free slot left                */

/* kernel-map build options (bit set) */
#define TS_KMAP_PAIRS 1u   /* also build per-offset (in, out) pair lists            */
#define TS_KMAP_BWD 2u     /* strided/target: also build the transposed relation    */
#define TS_KMAP_NATURAL 4u /* keep destination rows in index order inside tiles    */
#define TS_KMAP_TARGET 8u  /* outputs are caller-given coordinates (TargetConv3d)  */
#define TS_KMAP_TRANSPOSED 16u /* fine outputs of a transposed convolution      */
#define TS_KMAP_GROUPS 32u   /* also build per-tile pair groups (fetch on demand)   */
#define TS_KMAP_NO_TABLE 64u /* with TS_KMAP_GROUPS: no neighbour table or tile
                                lists for the forward relation (see ts_kmap_build) */

#define TS_TILE 16     /* destination rows per tile                  */
#define TS_GTILE 128   /* destination rows per pair-group tile        */
#define TS_MAX_KVOL 64 /* largest supported K^D                       */

/* Human-readable name of a status code (static string). */
const char* ts_status_string(ts_status s);

/* Library version string and the GPU architecture it was built for. */
const char* ts_version(void);

/* ------------------------------------------------------------------------
 * Coordinate hash (the "hashing" and "coordinate query" kernels of the
 * torch-lattice page, section "What remains familiar"; table size set by the
 * reserve ratio of section "Backend and configuration differences").
 *
 * The table maps a coordinate to a row index.  Internally voxels are grouped
 * in blocks (4x4x4 in 3-D, 8x8 in 2-D): an open-addressing table of `cap`
 * block slots, each owning the rows of its block's 64 cells, in one caller
 * buffer of ts_hash_table_bytes(cap) bytes (256-byte aligned).  The slot
 * layout is internal and may differ between runs; only the lookup function is
 * defined.  `cap` bounds the number of distinct blocks, so cap >= n always
 * suffices; cap <= 2^25 (larger tables return TS_ERR_UNSUPPORTED).
 * ---------------------------------------------------------------------- */

/* Capacity for n keys at reserve ratio rsv (>= 1): the smallest power of two
 * >= max(64, ceil(rsv * n)).  Returns -1 for n < 0 or rsv < 1. */
int64_t ts_hash_capacity(int64_t n, double rsv_ratio);

/* Bytes of a table of `cap` block slots (8 + 256 per slot).  A table buffer
 * must be zero-filled before its first build (an all-zero buffer is the
 * empty table); every build and every strided support then leaves it in a
 * state the next one clears itself, so one buffer can be rebuilt any number
 * of times with the same cap.  A buffer holding anything else (or last built
 * with a larger cap) gives wrong lookups: zero it again first. */
size_t ts_hash_table_bytes(int64_t cap);

/* Build the table of `n` coordinate rows coords[n][ndim+1] (device int32):
 * key(coords[i]) -> i, the lowest row winning for repeated keys.  `table`
 * (device, ts_hash_table_bytes(cap) bytes, see above) is rebuilt in place:
 * the slots the previous build used are cleared first; cap must be a power
 * of two >= n.  err_flags (device uint32, may be NULL) receives
 * TS_FLAG_DUP / TS_FLAG_RANGE / TS_FLAG_FULL. */
ts_status ts_hash_build(const int32_t* coords, int64_t n, int ndim, void* table, int64_t cap,
                        uint32_t* err_flags, hipStream_t stream);

/* rows[k] = row owning coordinate q[k] (device int32 [m][ndim+1]) or -1. */
ts_status ts_hash_query(const void* table, int64_t cap, int ndim, const int32_t* q, int64_t m,
                        int32_t* rows, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Downsampled support of a strided convolution (page section "Convolution
 * mapping": a strided forward convolution creates a downsampled support).
 *
 * Output coordinates are unique((b, floor(x/s), floor(y/s)[, floor(z/s)]))
 * over the input rows (floor toward -inf), ordered by first occurrence in
 * input row order.  out_coords (device int32, capacity n_in rows) receives
 * them, *n_out (device int64) their count, and out_table (device,
 * ts_hash_table_bytes(out_cap), out_cap a power of two >= n_in, zero-filled
 * before its first use like any table buffer) maps each
 * output coordinate to its output row -- it serves as the input table of a
 * following layer.  `scratch` (device) needs ts_support_scratch_bytes(n_in).
 * ---------------------------------------------------------------------- */
size_t ts_support_scratch_bytes(int64_t n_in);
ts_status ts_strided_support(const int32_t* in_coords, int64_t n_in, int ndim, int stride,
                             int32_t* out_coords, int64_t* n_out, void* out_table, int64_t out_cap,
                             void* scratch, size_t scratch_bytes, uint32_t* err_flags,
                             hipStream_t stream);

/* ------------------------------------------------------------------------
 * Generated support of a stride-1 convolution (torch-lattice migration page,
 * table "What is intentionally different", row on convolution intent: a
 * Conv3d generates its output support, unlike SubmConv3d).
 *
 * The outputs are every site q = c_i - delta_o that an input row i reaches
 * through a kernel offset o -- the sites whose window holds at least one
 * input -- each once, in order of first occurrence over (i ascending, then o
 * ascending).  Rows repeating an earlier coordinate add nothing; an
 * out-of-range input raises TS_FLAG_RANGE; sites outside the packable range
 * are not generated.  out_coords (device int32, n_out_cap rows) receives the
 * sites and *n_out (device int64) their count, clamped to n_out_cap: sites
 * past the capacity are dropped and raise TS_FLAG_FULL (n_in * ksize^ndim
 * rows always suffice).  out_table (out_cap a power of two, zero-filled
 * before its first use like any table buffer; a full table raises
 * TS_FLAG_FULL) maps each site to its output row.  `scratch` (device) needs
 * ts_generative_scratch_bytes(n_in, ndim, ksize).  The map over these outputs
 * is a TS_KMAP_TARGET map at stride 1, with out_table for its transposed
 * relation.
 * ---------------------------------------------------------------------- */
/* Scratch of ts_generative_support and ts_transposed_support (both hold
 * three words per (input row, offset) candidate plus a scan). */
size_t ts_generative_scratch_bytes(int64_t n_in, int ndim, int ksize);
ts_status ts_generative_support(const int32_t* in_coords, int64_t n_in, int ndim, int ksize,
                                int32_t* out_coords, int64_t n_out_cap, int64_t* n_out,
                                void* out_table, int64_t out_cap, void* scratch, size_t scratch_bytes,
                                uint32_t* err_flags, hipStream_t stream);

/* Generated support of a transposed convolution of stride s (torch-lattice
 * migration page, "Convolution mapping" table: GenerativeConvTranspose3d
 * generates output support, where ConvTranspose3d reuses a relation).  The
 * outputs are every fine site s*c_j + delta_o that a (coarse) input row j
 * reaches through offset o, each once, in order of first occurrence over
 * (j ascending, then o ascending); for k = s these are the s^D children of
 * every input.  Repeats, range, capacity, table and scratch behave as in
 * ts_generative_support.  The map over these outputs is a TS_KMAP_TRANSPOSED
 * map with this out_table. */
ts_status ts_transposed_support(const int32_t* in_coords, int64_t n_in, int ndim, int ksize, int stride,
                                int32_t* out_coords, int64_t n_out_cap, int64_t* n_out,
                                void* out_table, int64_t out_cap, void* scratch, size_t scratch_bytes,
                                uint32_t* err_flags, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Voxelization and devoxelization (torch-lattice page, "What remains
 * familiar": the CUDA kernels cover voxelization and devoxelization).
 *
 * Point i (batch[i], or 0 when batch is NULL; position pos[i][ndim], device
 * float32) goes to voxel floor((pos - origin) / size) per axis, decided in
 * float32: a rounded subtraction, a division rounded to nearest even and a
 * floor (size and origin are host arrays of ndim floats; size > 0).  A point
 * whose voxel or batch leaves the packable range is dropped (vox_of = -1)
 * and raises TS_FLAG_RANGE.  Voxels are numbered in order of first
 * occurrence over the points: out_coords (device int32, capacity n rows)
 * receives them, *n_out (device int64) their count, vox_of[n] (device) each
 * point's voxel row, and out_table (zero-filled before its first use, out_cap
 * a power of two) maps each voxel to its row, so it serves as the input
 * table of a kernel map without a hash build.  With feats (device
 * [n][c] float32; may be NULL), out_feats (device [n][c] float32) receives
 * the mean of each voxel's point features in its first *n_out rows; the sums
 * use float atomics, so their order (and the last bits) may vary between
 * runs.  scratch (device) needs ts_voxelize_scratch_bytes(n).
 * ---------------------------------------------------------------------- */
size_t ts_voxelize_scratch_bytes(int64_t n_points);
ts_status ts_voxelize(const int32_t* batch, const float* pos, int64_t n, int ndim, const float* size,
                      const float* origin, const float* feats, int c, int32_t* out_coords, int64_t* n_out,
                      void* out_table, int64_t out_cap, int32_t* vox_of, float* out_feats, void* scratch,
                      size_t scratch_bytes, uint32_t* err_flags, hipStream_t stream);

/* Devoxelization: point_feats[i] = vox_feats[vox_of[i]] ([n][c], any feature
 * type), or zeros for a dropped point (vox_of[i] = -1). */
ts_status ts_devoxelize(const int32_t* vox_of, int64_t n, const void* vox_feats, int c, void* point_feats,
                        ts_dtype dtype, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Kernel map (the "kernel-map construction" of the page's section "Sparse
 * tensor expectations"): for every output row j and offset o, the input row
 * i at q_j + delta_o (stride 1) or s q_j + delta_o (stride s), as a relation
 * between destination rows and source rows:
 *
 *   nbr[d*kvol + o] is the source row of destination row d at offset o, or
 *   -1; row_mask[d] has bit o set exactly when nbr[d*kvol + o] >= 0.  Both
 *   cover the destination rows below the device count n_dest; past it,
 *   row_mask is 0 and nbr is left unwritten.
 *   Destination rows are grouped in tiles of TS_TILE: tile_rows[t*TS_TILE + r]
 *   is the destination row in slot r of tile t (-1 for padding; every row
 *   appears once), and tile_mask[t] is the OR of its rows' masks, so the
 *   contraction of a tile skips every offset none of its rows uses.
 *
 * Which destination rows share a tile is a performance choice (rows with
 * similar masks are grouped unless TS_KMAP_NATURAL is set); the relation
 * itself -- the set of (in, out, offset) triples -- is fixed.
 *
 * Pair groups (TS_KMAP_GROUPS; the layout the fetch-on-demand dataflow
 * reads): destination rows are cut into group tiles of TS_GTILE consecutive
 * rows; tile t owns kvol * TS_GTILE entries of gsrc / gslot starting at
 * t * kvol * TS_GTILE.  gcount[t*kvol + o] is the number of pairs of tile t
 * at offset o.  Inside the tile, offset o's pairs are listed in destination
 * order (gslot = destination row - t * TS_GTILE, gsrc = its source row),
 * starting at entry 16 * sum_{o' < o} ceil(gcount[t*kvol + o'] / 16): each
 * offset's run is padded to whole groups of 16 (padding entries hold
 * gsrc = -1 and gslot = TS_GTILE), so group g of the tile is entries
 * [16g, 16g + 16).  Entries past a tile's last group are not written.
 * ---------------------------------------------------------------------- */
typedef struct ts_rel {
  int64_t n_dest_cap;    /* destination rows, upper bound (host)               */
  int64_t n_tiles;       /* ceil(n_dest_cap / TS_TILE)                         */
  const int64_t* n_dest; /* device int64: destination row count                */
  uint64_t* tile_mask;   /* device [n_tiles] (NULL without the table)          */
  int32_t* tile_rows;    /* device [n_tiles * TS_TILE] (NULL without the table) */
  int32_t* nbr;          /* device [n_dest_cap * kvol] (NULL without the table) */
  uint64_t* row_mask;    /* device [n_dest_cap]                                */
  int64_t n_gtiles;      /* ceil(n_dest_cap / TS_GTILE), 0 without groups       */
  int32_t* gcount;       /* device [n_gtiles * kvol]                           */
  int32_t* gsrc;         /* device [n_gtiles * kvol * TS_GTILE]                */
  uint8_t* gslot;        /* device [n_gtiles * kvol * TS_GTILE]                */
} ts_rel;

typedef struct ts_kmap {
  int32_t ndim, ksize, stride, kvol;
  uint32_t flags;      /* TS_KMAP_* bits actually built                            */
  int32_t mirror_bwd;  /* 1: the transposed relation is fwd with offset kvol-1-o  */
  int64_t n_in;        /* input rows                                               */
  int64_t n_out_cap;   /* output rows, upper bound                                 */
  int64_t* n_out;      /* device int64: output rows                                */
  ts_rel fwd;          /* destination = output rows, source = input rows           */
  ts_rel bwd;          /* strided/target with TS_KMAP_BWD: destination = input rows */
  int64_t pair_cap;    /* capacity of the pair lists                               */
  int64_t* pair_start; /* device [kvol+1]: offset o owns pairs [start[o], start[o+1]) */
  int32_t* pair_in;    /* device [pair_cap] input row of each pair, output-row order */
  int32_t* pair_out;   /* device [pair_cap] output row of each pair                  */
  void* scratch;       /* device scratch inside the map buffer                     */
  size_t scratch_bytes;
} ts_kmap;

/* Bytes of the map buffer for the given shape and TS_KMAP_* flags. */
size_t ts_kmap_bytes(int64_t n_in, int64_t n_out_cap, int ndim, int ksize, int stride, uint32_t flags);

/* Build the kernel map into `buf` (device, ts_kmap_bytes(...) bytes) and fill
 * the host struct *map with pointers into it.
 *   stride == 1 (submanifold): ksize odd; the outputs are the inputs, so
 *     out_coords / n_out / out_table may be NULL and n_out_cap = n_in.  An
 *     output row takes part only if it owns its coordinate in in_table.
 *   stride > 1: out_coords (device, n_out_cap rows), n_out (device int64)
 *     and, with TS_KMAP_BWD, out_table (out_cap slots) describe the output
 *     support, normally from ts_strided_support (distinct coordinates).
 *   TS_KMAP_TARGET (convolution at caller-given output coordinates, the
 *     TargetConv3d of the torch-lattice migration page, tables "What is
 *     intentionally different" and "Convolution mapping"): out_coords /
 *     n_out_cap / n_out are the caller's targets, which need not be inputs
 *     and may repeat; output row j takes the input at s*q_j + delta_o (s = 1
 *     included) for every offset o, with any ksize.  A target row whose
 *     coordinate is outside the packable range takes no inputs.  Repeated
 *     targets are fine for the forward pass and wgrad; dgrad needs distinct
 *     targets (its scatter into input rows assumes each input meets an
 *     offset once), and its transposed relation (TS_KMAP_BWD) needs
 *     out_table = the ts_hash_build table of the targets (or the table
 *     ts_generative_support leaves).
 *   TS_KMAP_TRANSPOSED (a transposed convolution onto generated or given fine
 *     coordinates, e.g. from ts_transposed_support): out_coords / n_out_cap /
 *     n_out are the fine outputs and out_table their table (required: an
 *     output row takes part only if it owns its coordinate there); output
 *     row j takes the coarse input at (p_j - delta_o)/s for every offset o
 *     where that divides exactly -- the strided relation read the other way.
 *     With TS_KMAP_BWD the transposed relation (coarse rows to fine rows, the
 *     strided relation itself) is built too, for dgrad.
 * in_table / in_cap is the ts_hash_build table of the inputs.
 *   TS_KMAP_GROUPS builds the pair groups of every relation the map holds
 *     (the forward one, and the transposed one with TS_KMAP_BWD);
 *     TS_KMAP_NO_TABLE then leaves out the forward relation's neighbour
 *     table, tile lists and tile masks (NULL in map->fwd) where its probe
 *     emits the groups directly -- submanifold and strided maps of kernel
 *     size 1, 2 or 3 in 3-D and 2, 3 or 5 in 2-D; other shapes keep the table.
 *     A map without the table serves the fetch-on-demand and gather-scatter
 *     dataflows and wgrad; the other dataflows and pooling need the table
 *     and return TS_ERR_INVALID_ARG on it.  TS_KMAP_NO_TABLE without
 *     TS_KMAP_GROUPS is TS_ERR_INVALID_ARG. */
ts_status ts_kmap_build(const int32_t* in_coords, int64_t n_in, const void* in_table, int64_t in_cap,
                        const int32_t* out_coords, int64_t n_out_cap, const int64_t* n_out,
                        const void* out_table, int64_t out_cap, int ndim, int ksize, int stride,
                        uint32_t flags, void* buf, size_t buf_bytes, ts_kmap* map, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Convolution (forward, dgrad, wgrad) over a built map.  Features are
 * fp32 / fp16 / bf16 with fp32 accumulation; the output type is fp32 or the
 * input type (round to nearest even).  Every output row is written exactly
 * once (rows without neighbours get zeros); there are no atomics, so results
 * are bitwise repeatable.
 * ---------------------------------------------------------------------- */
#define TS_OP_FWD 0
#define TS_OP_DGRAD 1
#define TS_OP_WGRAD 2
#define TS_OP_TRANSPOSE 3

/* Workspace bytes for an op on this map (0 is a valid answer). */
size_t ts_conv_workspace_bytes(const ts_kmap* map, int cin, int cout, int op, ts_dtype in_dtype,
                               ts_dataflow dataflow);

/* Packs w[kvol][cin][cout] (the layer's weights, fp16 or bf16, device) into
 * ws in the fragment order the implicit GEMM of `op` reads (TS_OP_FWD,
 * TS_OP_DGRAD or TS_OP_TRANSPOSE on this map: dgrad and the transposed
 * convolution mirror the offsets on a submanifold map, dgrad also swaps the
 * channel roles).  Without it the implicit-GEMM calls either read the
 * weights as stored (forward-layout weights on 16-byte-aligned storage, for
 * the shapes where that is faster) or pack them into ws as their first
 * launch; packing separately lets a caller whose weights stay fixed pack once
 * (on any stream: it needs only the weights, not the map's contents) and
 * then call the op with TS_DATAFLOW_IMPLICIT_GEMM_PACKED and the same ws,
 * cin, cout and dtype.
 * ws_bytes must be at least ts_conv_workspace_bytes(map, cin, cout, op,
 * in_dtype, TS_DATAFLOW_IMPLICIT_GEMM).  Errors: TS_ERR_INVALID_ARG (null,
 * bad op or sizes, short ws), TS_ERR_UNSUPPORTED (the shape or dtype has no
 * implicit GEMM: fp32, channels not multiples of 32 / 16, kvol > 28). */
ts_status ts_conv_pack_weights(const ts_kmap* map, const void* w, int cin, int cout, int op, ts_dtype in_dtype,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/* Sparse convolution forward over a built map (torch-lattice migration page,
 * section "Sparse tensor expectations": coordinate row i owns feature row i
 * and the kernel map relates them; section "Backend and configuration
 * differences": every dataflow computes the same result for a fixed relation
 * and weight tensor, up to floating-point rounding; TorchSparse++ abstract:
 * the gather-GEMM-scatter and implicit-GEMM dataflows).
 *   y[j][co] = sum over the map's triples (i, j, o) of sum_ci x[i][ci] w[o][ci][co]
 * x: device [map->n_in][cin] (row-major, in_dtype); w: device [kvol][cin][cout]
 * (in_dtype); y: device [n_out_cap][cout] (out_dtype), every row below the
 * device output count written once (zeros for rows without pairs), rows at or
 * past it not written.  `dataflow` picks the kernel (AUTO: per shape); ws
 * (device, may be NULL when ts_conv_workspace_bytes(map, cin, cout,
 * TS_OP_FWD, in_dtype, dataflow) is 0) is scratch the caller owns.  Errors:
 * TS_ERR_INVALID_ARG (null or short buffers, channel counts outside
 * [1, 65536], a dataflow the map lacks the lists for), TS_ERR_UNSUPPORTED
 * (an output type other than fp32 or in_dtype; packed weights for a shape
 * without an implicit GEMM), TS_ERR_HIP (launch failure).  Any stride. */
ts_status ts_conv_fwd(const ts_kmap* map, const void* x, int cin, const void* w, int cout, void* y,
                      ts_dtype in_dtype, ts_dtype out_dtype, ts_dataflow dataflow, void* ws,
                      size_t ws_bytes, hipStream_t stream);

/* Submanifold SubmConv3d / SubmConv2d forward (torch-lattice migration page,
 * "Convolution mapping" table: SubmConv3d preserves the input coordinate
 * support; "What is intentionally different", convolution intent): the
 * output rows are the input rows, y[n_in][cout].  Arguments, ownership and
 * errors as ts_conv_fwd; a map that is not submanifold (stride > 1, a
 * TS_KMAP_TARGET or TS_KMAP_TRANSPOSED map) returns TS_ERR_INVALID_ARG. */
ts_status ts_subm_conv_fwd(const ts_kmap* map, const void* x, int cin, const void* w, int cout, void* y,
                           ts_dtype in_dtype, ts_dtype out_dtype, ts_dataflow dataflow, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/* Strided Conv3d / Conv2d forward, support generation included
 * (torch-lattice migration page, "Convolution mapping" table: a strided
 * forward convolution creates a downsampled support): runs
 * ts_strided_support, ts_kmap_build (kmap_flags) and ts_conv_fwd in order.
 * Errors of any of the three are returned before the later ones launch;
 * every argument is validated before the first launch.
 * `map_buf` holds ts_kmap_bytes(n_in, n_in, ndim, ksize, stride, kmap_flags)
 * + ts_support_scratch_bytes(n_in) bytes; *map is filled for the backward
 * pass.  y has capacity n_in rows; rows >= *n_out are not written. */
ts_status ts_conv_fwd_strided(const int32_t* in_coords, int64_t n_in, int ndim, const void* in_table,
                              int64_t in_cap, int ksize, int stride, uint32_t kmap_flags,
                              int32_t* out_coords, int64_t* n_out, void* out_table, int64_t out_cap,
                              uint32_t* err_flags, void* map_buf, size_t map_bytes, ts_kmap* map,
                              const void* x, int cin, const void* w, int cout, void* y,
                              ts_dtype in_dtype, ts_dtype out_dtype, ts_dataflow dataflow, void* ws,
                              size_t ws_bytes, hipStream_t stream);

/* Generative stride-1 Conv3d / Conv2d forward, support generation included:
 * runs ts_generative_support, ts_kmap_build (kmap_flags | TS_KMAP_TARGET,
 * stride 1) and ts_conv_fwd in order.  `map_buf` holds
 * ts_kmap_bytes(n_in, n_out_cap, ndim, ksize, 1, kmap_flags | TS_KMAP_TARGET)
 * + ts_generative_scratch_bytes(n_in, ndim, ksize) bytes; *map is filled for
 * the backward pass.  y has n_out_cap rows; rows >= *n_out are not written. */
ts_status ts_conv_fwd_generative(const int32_t* in_coords, int64_t n_in, int ndim, const void* in_table,
                                 int64_t in_cap, int ksize, uint32_t kmap_flags, int32_t* out_coords,
                                 int64_t n_out_cap, int64_t* n_out, void* out_table, int64_t out_cap,
                                 uint32_t* err_flags, void* map_buf, size_t map_bytes, ts_kmap* map,
                                 const void* x, int cin, const void* w, int cout, void* y,
                                 ts_dtype in_dtype, ts_dtype out_dtype, ts_dataflow dataflow, void* ws,
                                 size_t ws_bytes, hipStream_t stream);

/* ConvTranspose3d / ConvTranspose2d over an existing relation (torch-lattice
 * migration page, "Convolution mapping": a transposed convolution that
 * consumes an existing relation): y[n_in][cout] = sum over the map's triples
 * (i, j, o) of x[j] . W[o], with x[n_out][cin] on the map's outputs and
 * W[kvol][cin][cout] -- the relation of dgrad, the weights as the forward
 * reads them.  Strided maps need TS_KMAP_BWD (implicit GEMM) or TS_KMAP_PAIRS
 * (gather-scatter); a submanifold map uses its mirrored offsets.  Workspace:
 * ts_conv_workspace_bytes(map, cin, cout, TS_OP_TRANSPOSE, ...). */
ts_status ts_conv_transpose_fwd(const ts_kmap* map, const void* x, int cin, const void* w, int cout, void* y,
                                ts_dtype in_dtype, ts_dtype out_dtype, ts_dataflow dataflow, void* ws,
                                size_t ws_bytes, hipStream_t stream);

/* Sparse pooling over a kernel map (torch-lattice page, "What remains
 * familiar": the CUDA kernels cover pooling, over the same maps as
 * convolution): y[n_out][c] = the maximum (TS_POOL_MAX) or the mean
 * (TS_POOL_AVG) of x[i] over the map's triples (i, j, o) of output row j --
 * the inputs present in the window, not K^D -- and 0 for an output with
 * none.  x is [n_in][c] (fp32/fp16/bf16), y fp32 or the input type; the
 * maximum is exact in either, the mean is accumulated in fp32 and rounded to
 * nearest even.  Rows of y at or past *n_out are not written. */
#define TS_POOL_MAX 0
#define TS_POOL_AVG 1
ts_status ts_pool_fwd(const ts_kmap* map, const void* x, int c, void* y, ts_dtype in_dtype, ts_dtype out_dtype,
                      int mode, hipStream_t stream);

/* Relational graph convolution (TorchSparse++ abstract: the library also runs
 * graph convolutions; sparse convolution is the case "edges = kernel-map
 * triples, relations = offsets").  Edges are grouped by destination (CSR):
 * node v owns edges [indptr[v], indptr[v+1]) (device int64 [n_dst+1]), edge
 * e runs from src[e] (device int32, < n_src) with relation rel[e] (device
 * int32, < n_rel).  y[n_dst][cout] = sum over v's edges of x[src] . w[rel]
 * with x [n_src][cin], w [n_rel][cin][cout] and fp32 accumulation in edge
 * order (so the result does not vary between runs); no normalisation; 0 for
 * a node without edges.  An edge with an out-of-range source or relation is
 * skipped and raises TS_FLAG_RANGE.  y is fp32 or the input type. */
ts_status ts_graph_conv_fwd(const int64_t* indptr, const int32_t* src, const int32_t* rel, int64_t n_dst,
                            int64_t n_src, int n_rel, const void* x, int cin, const void* w, int cout, void* y,
                            ts_dtype in_dtype, ts_dtype out_dtype, uint32_t* err_flags, hipStream_t stream);

/* Input gradient of the forward (the training workloads of the TorchSparse++
 * abstract; the adjoint of ts_conv_fwd over the same relation):
 *   dx[i][ci] = sum over triples (i, j, o) of sum_co dy[j][co] w[o][ci][co]
 * dy: device [n_out_cap][cout]; w as in the forward; dx: device
 * [n_in][cin] (out_dtype), every row written once.  A submanifold map uses
 * its own offsets mirrored ((i, j, o) and (j, i, kvol-1-o) are the same
 * pair); strided and target maps need TS_KMAP_BWD (implicit GEMM) or
 * TS_KMAP_PAIRS (gather-scatter), else TS_ERR_INVALID_ARG.  Workspace and
 * errors as ts_conv_fwd with TS_OP_DGRAD. */
ts_status ts_conv_bwd_dgrad(const ts_kmap* map, const void* dy, int cout, const void* w, int cin, void* dx,
                            ts_dtype in_dtype, ts_dtype out_dtype, ts_dataflow dataflow, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/* Weight gradient of the forward (the training workloads of the TorchSparse++
 * abstract; the adjoint of ts_conv_fwd in w):
 *   dw[o][ci][co] = sum over triples (i, j, o) of x[i][ci] dy[j][co]
 * x: device [n_in][cin], dy: device [n_out_cap][cout] (in_dtype); dw: device
 * fp32 [kvol][cin][cout], overwritten.  Needs TS_KMAP_PAIRS (else
 * TS_ERR_INVALID_ARG); ws (device) holds ts_conv_workspace_bytes(map, cin,
 * cout, TS_OP_WGRAD, ...) bytes.  The per-offset reduction is split over
 * chunks of pairs and summed in a fixed order, so the result is the same
 * bits on every run. */
ts_status ts_conv_bwd_wgrad(const ts_kmap* map, const void* x, int cin, const void* dy, int cout,
                            ts_dtype in_dtype, float* dw, void* ws, size_t ws_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * ts_conv_bwd_dgrad with the implicit GEMM's packed weights in a static
 * device array of the library instead of a caller workspace, so the call
 * allocates nothing.  The array holds TS_NOALLOC_SCRATCH_BYTES; each GPU the
 * library runs on keeps its own copy until the process ends.  Dataflow: the
 * implicit GEMM where the shape has one (fp16/bf16, source channels a
 * multiple of 32 up to 128, destination channels a multiple of 16), else the
 * direct kernel, which needs no scratch; the gather-scatter dataflow is not
 * offered (its accumulator grows with the rows).  Arguments, results and the
 * other errors are those of ts_conv_bwd_dgrad; a shape whose packed weights
 * exceed TS_NOALLOC_SCRATCH_BYTES returns TS_ERR_UNSUPPORTED, and a failed
 * lookup of the array's device address TS_ERR_HIP.  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (unordered streams,
 * host threads) race and give wrong results; order them on one stream. */
#define TS_NOALLOC_SCRATCH_BYTES (4u << 20)
ts_status ts_conv_bwd_dgrad_noalloc(const ts_kmap* map, const void* dy, int cout, const void* w, int cin, void* dx,
                                    ts_dtype in_dtype, ts_dtype out_dtype, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Bounds-check build.  The library also builds as libts_debug.so, compiled
 * with TS_DEBUG_CHECKS: there the contraction, pooling and weight-gradient
 * kernels check every row index they read from a map (neighbour entries,
 * tile rows, pair lists, pair-group entries and slots) against the matrix it
 * indexes.  An index out of range is replaced by one inside, so no access
 * leaves the caller's buffers, and raises a bit below; the results of that
 * call are then meaningless.  Everything else is the regular library.
 *
 * ts_debug_violations waits for the current device (hipDeviceSynchronize),
 * ORs the bits raised on it since the previous call into *bits (host) and
 * clears them.  Errors: TS_ERR_INVALID_ARG (bits NULL), TS_ERR_HIP (the wait
 * or a copy failed), TS_ERR_UNSUPPORTED in the regular build, which has no
 * checks.
 * ---------------------------------------------------------------------- */
#define TS_DEBUG_SRC_ROW 1u /* a source row index outside the source matrix                 */
#define TS_DEBUG_DST_ROW 2u /* a destination row, pair-group slot or group count out of range */
ts_status ts_debug_violations(uint32_t* bits);

#ifdef __cplusplus
}
#endif

#endif /* TS_H_ */
