/*
 * qmoe_oracle.c -- plain, slow CPU reference of the quantized MoE (QMoE) FFN
 * layer, in double precision.
 *
 * TEST INFRASTRUCTURE.  This is the oracle the GPU library is checked
 * against.  Only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark load it.  It shares no code, header, table or helper with the
 * GPU library, and neither side calls the other.
 *
 * Sources (page title, then the function / paragraph followed):
 *   [qmoe.rs]   docs.rs source page of onnx-runtime-ep-cuda, src/kernels/qmoe.rs
 *   [PR 32198]  onnxruntime pull request 32198, "[CUDA] QMoE: fused int2
 *               mixed-input GEMM + GeGLU activation + fractional zero-point"
 *   [PR 33569]  onnxruntime pull request 33569, "[CUDA] Add fast INT3 QMoE
 *               kernels and offline SM80 INT2/INT4 prepack support"
 *   [gemm_quant_moe.rs]  metrale_model_layers layers/ops/gemm_quant_moe.rs
 *
 * Every function computes the plain definition.  No blocking, no fusion, no
 * reordering: routing is a full sort, the projections are per-route dot
 * products over a freshly dequantized weight row.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - 3-bit codes: 8 codes per 3-byte group, code j = bits [3j, 3j+3) of the
 *     little-endian 24-bit word ([PR 33569] describes 24-bit 8-code groups).
 *   - 3-bit zero-point tensors hold one byte per block.
 *   - fc1 rows are gate/up interleaved: row 2j is the gate, 2j+1 the up row.
 *   - scales have the activation dtype (fp16 or bf16).
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -fPIC -shared (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F16 1
#define ORACLE_BF16 2
#define ORACLE_SWIGLU 0
#define ORACLE_GEGLU 1

/* ------------------------------------------------------------------ */
/* fp16 / bf16 widening, written from the IEEE binary16 definition and */
/* from bf16 being the top half of a binary32.                         */
/* ------------------------------------------------------------------ */
static double widen_f16(uint16_t h)
{
    const int negative = (h >> 15) & 1;
    const int exponent = (h >> 10) & 0x1f;
    const int fraction = h & 0x3ff;
    double magnitude;
    if (exponent == 0) {
        magnitude = ldexp((double)fraction, -24);               /* subnormal */
    } else if (exponent == 31) {
        magnitude = fraction ? NAN : INFINITY;
    } else {
        magnitude = ldexp((double)(1024 + fraction), exponent - 25);
    }
    return negative ? -magnitude : magnitude;
}

static double widen_bf16(uint16_t b)
{
    const uint32_t word = (uint32_t)b << 16;
    float f;
    memcpy(&f, &word, sizeof f);
    return (double)f;
}

static double widen(uint16_t bits, int dtype)
{
    return dtype == ORACLE_BF16 ? widen_bf16(bits) : widen_f16(bits);
}

void oracle_widen(const uint16_t* bits, int64_t n, int32_t dtype, double* out)
{
    for (int64_t i = 0; i < n; ++i) {
        out[i] = widen(bits[i], dtype);
    }
}

/* ------------------------------------------------------------------ */
/* Routing  [qmoe.rs, total_order_key / route_value_is_better /         */
/* qmoe_route softmax weighting]                                        */
/* ------------------------------------------------------------------ */

/* The route key orders float32 bit patterns totally: non-negative floats
 * keep their bits as a signed integer; for negative floats the magnitude
 * bits are flipped so that larger magnitudes rank lower.  -0 sorts below
 * +0, +NaN above +inf, -NaN below -inf. */
static int32_t route_key(float logit)
{
    int32_t bits;
    memcpy(&bits, &logit, sizeof bits);
    return bits < 0 ? (int32_t)(bits ^ 0x7fffffff) : bits;
}

int32_t oracle_route_key(float logit) { return route_key(logit); }

typedef struct {
    int32_t key;
    int32_t expert;
} ranked_expert;

/* Higher key first; equal keys: lower expert index first. */
static int rank_order(const void* a, const void* b)
{
    const ranked_expert* x = (const ranked_expert*)a;
    const ranked_expert* y = (const ranked_expert*)b;
    if (x->key != y->key) {
        return x->key > y->key ? -1 : 1;
    }
    return (x->expert > y->expert) - (x->expert < y->expert);
}

/* One token: the top_k experts in descending key order, and their weights.
 * m is the largest non-NaN logit (NaN entries are skipped, as a running
 * fmax does; -inf if there is none).  Each selected expert's numerator is
 * exp(l - m); the denominator is the sum of the selected numerators when
 * normalize is set, otherwise the sum of exp(l - m) over every expert.
 * With an aggregation row (the operator's router_weights input, [qmoe.rs,
 * qmoe_route, its router_weights branch]) the logits only select: a
 * selected expert's weight is its aggregation value, divided by the sum of
 * the selected values when normalize is set, and 0 when that sum is 0. */
static void route_one(const float* logits, const float* aggregation, int32_t E, int32_t top_k,
                      int32_t normalize, ranked_expert* scratch, int32_t* ids, double* weights)
{
    for (int32_t e = 0; e < E; ++e) {
        scratch[e].key = route_key(logits[e]);
        scratch[e].expert = e;
    }
    qsort(scratch, (size_t)E, sizeof(ranked_expert), rank_order);

    if (aggregation) {
        double sum = 0.0;
        for (int32_t s = 0; s < top_k; ++s) {
            ids[s] = scratch[s].expert;
            sum += (double)aggregation[ids[s]];
        }
        const double denominator = normalize ? sum : 1.0;
        for (int32_t s = 0; s < top_k; ++s) {
            weights[s] = denominator == 0.0 ? 0.0 : (double)aggregation[ids[s]] / denominator;
        }
        return;
    }

    double m = -INFINITY;
    for (int32_t e = 0; e < E; ++e) {
        const double l = (double)logits[e];
        if (!isnan(l) && l > m) {
            m = l;
        }
    }
    double denominator = 0.0;
    for (int32_t s = 0; s < top_k; ++s) {
        ids[s] = scratch[s].expert;
        weights[s] = exp((double)logits[ids[s]] - m);
        if (normalize) {
            denominator += weights[s];
        }
    }
    if (!normalize) {
        for (int32_t e = 0; e < E; ++e) {
            denominator += exp((double)logits[e] - m);
        }
    }
    for (int32_t s = 0; s < top_k; ++s) {
        weights[s] /= denominator;
    }
}

void oracle_route(const float* logits, const float* router_weights, int64_t T, int32_t E,
                  int32_t top_k, int32_t normalize, int32_t* ids, double* weights)
{
#pragma omp parallel
    {
        ranked_expert* scratch = (ranked_expert*)malloc(sizeof(ranked_expert) * (size_t)E);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            route_one(logits + t * E, router_weights ? router_weights + t * E : NULL, E, top_k,
                      normalize, scratch, ids + t * top_k, weights + t * top_k);
        }
        free(scratch);
    }
}

/* ------------------------------------------------------------------ */
/* Router projection  [gemm_quant_moe.rs, moe_gate_topk_fused: the gate   */
/* logits of a token are its input row times the transposed gate weight   */
/* matrix, one logit per expert; ferrum moe.rs, the router GEMM before    */
/* routing].  logits[t, e] = sum_h x[t, h] * w[e, h], exact in double     */
/* from the dtype values (w is [E, H] row-major).                         */
/* ------------------------------------------------------------------ */
void oracle_router_logits(const uint16_t* hidden, const uint16_t* weight, int64_t T, int32_t H,
                          int32_t E, int32_t dtype, double* logits)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int32_t h = 0; h < H; ++h) {
                acc += widen(hidden[t * H + h], dtype) * widen(weight[(int64_t)e * H + h], dtype);
            }
            logits[t * E + e] = acc;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Codes, zero points, dequantization                                   */
/* [qmoe.rs, decode_affine_weight]; [PR 32198, zero_point_offset];      */
/* [PR 33569, 24-bit 8-code INT3 groups]                                */
/* ------------------------------------------------------------------ */

/* Code number kk of one packed row.  2- and 4-bit codes fill each byte from
 * the least significant bits up; 3-bit codes come in 3-byte groups of 8. */
static int code_at(const uint8_t* row, int64_t kk, int bits)
{
    if (bits == 3) {
        const uint8_t* group = row + (kk / 8) * 3;
        const uint32_t word = (uint32_t)group[0] | ((uint32_t)group[1] << 8)
                              | ((uint32_t)group[2] << 16);
        return (int)((word >> (3 * (kk % 8))) & 7u);
    }
    const int per_byte = 8 / bits;
    return (row[kk / per_byte] >> ((kk % per_byte) * bits)) & ((1 << bits) - 1);
}

static int64_t zero_point_row_bytes(int64_t n_blocks, int bits)
{
    return bits == 3 ? n_blocks : (n_blocks + (8 / bits) - 1) / (8 / bits);
}

/* Zero point of one quantization block: a uint8 tensor entry if given (it
 * takes precedence), else the fractional offset if it is not NaN, else the
 * symmetric centre 2^(bits-1). */
static double zero_point_of(const uint8_t* zp_row, int64_t block, int bits, double zpo)
{
    if (zp_row) {
        if (bits == 3) {
            return (double)zp_row[block];
        }
        const int per_byte = 8 / bits;
        return (double)((zp_row[block / per_byte] >> ((block % per_byte) * bits))
                        & ((1 << bits) - 1));
    }
    if (!isnan(zpo)) {
        return zpo;
    }
    return (double)(1 << (bits - 1));
}

/* One dequantized row W[n, 0..K) = (code - zp) * scale, exact in double. */
static void dequant_row(const uint8_t* codes, const uint16_t* scales, const uint8_t* zero_points,
                        int64_t row, int32_t K, int32_t bits, int32_t block_size, double zpo,
                        int32_t dtype, int32_t* q_out, double* w_out)
{
    const int64_t row_bytes = (int64_t)K * bits / 8;
    const int64_t n_blocks = K / block_size;
    const uint8_t* code_row = codes + row * row_bytes;
    const uint16_t* scale_row = scales + row * n_blocks;
    const uint8_t* zp_row =
        zero_points ? zero_points + row * zero_point_row_bytes(n_blocks, bits) : NULL;
    for (int64_t kk = 0; kk < K; ++kk) {
        const int64_t block = kk / block_size;
        const int q = code_at(code_row, kk, bits);
        if (q_out) {
            q_out[kk] = q;
        }
        if (w_out) {
            w_out[kk] = ((double)q - zero_point_of(zp_row, block, bits, zpo))
                        * widen(scale_row[block], dtype);
        }
    }
}

/* Dequantize `rows` packed rows of length K (any of q_out / w_out may be NULL). */
void oracle_dequant(const uint8_t* codes, const uint16_t* scales, const uint8_t* zero_points,
                    int64_t rows, int32_t K, int32_t bits, int32_t block_size, double zpo,
                    int32_t dtype, int32_t* q_out, double* w_out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        dequant_row(codes, scales, zero_points, r, K, bits, block_size, zpo, dtype,
                    q_out ? q_out + r * K : NULL, w_out ? w_out + r * K : NULL);
    }
}

/* ------------------------------------------------------------------ */
/* Gated activation  [qmoe.rs, qmoe_activate (tanh GELU constants) and  */
/* swiglu_value; PR 32198, GeGLU]                                       */
/* SwiGLU: the gate is bounded above by limit (fmin, so a NaN gate      */
/* becomes limit), the linear part clamped to [-limit, limit] unless it */
/* is NaN; value = g' * sigmoid(alpha g') * (u' + beta).  The defaults  */
/* alpha = 1, beta = 0, limit = +inf give silu(g) * u.  GeGLU uses the   */
/* tanh-GELU gate and takes no parameters.                              */
/* ------------------------------------------------------------------ */
typedef struct {
    double alpha, beta, limit;
} act_params;

static double gated(double gate, double up, int activation, const act_params* p)
{
    if (activation == ORACLE_GEGLU) {
        const double inner = 0.7978845608028654 * (gate + 0.044715 * gate * gate * gate);
        return 0.5 * gate * (1.0 + tanh(inner)) * up;
    }
    const double g = fmin(gate, p->limit);
    const double u = isnan(up) ? up : fmin(fmax(up, -p->limit), p->limit);
    return g / (1.0 + exp(-p->alpha * g)) * (u + p->beta);
}

double oracle_gated(double gate, double up, int32_t activation, double alpha, double beta,
                    double limit)
{
    const act_params p = {alpha, beta, limit};
    return gated(gate, up, activation, &p);
}

/* Options of the operator beyond the base layer [qmoe.rs, QMoEKernel and
 * its attributes]: expert biases added to the float32 projection outputs
 * (fc1 before the activation), the fc1 gate/up layout (swiglu_fusion 1:
 * interleaved rows 2j / 2j+1; 2: concatenated halves, gate j and up I + j;
 * 0: fc1 holds the I gate rows and a separate fc3 projection the I up
 * rows), the SwiGLU parameters, and router_weights for the routing
 * weights.  Every pointer may be NULL. */
typedef struct {
    const float* fc1_bias;       /* [E, rows of fc1] */
    const float* fc2_bias;       /* [E, H] */
    const uint8_t* fc3_codes;
    const uint16_t* fc3_scales;
    const uint8_t* fc3_zp;
    int32_t fc3_bits;
    const float* fc3_bias;       /* [E, I] */
    const float* router_weights; /* [T, E] */
    int32_t swiglu_fusion;
    double alpha, beta, limit;
} oracle_opts;

/* ------------------------------------------------------------------ */
/* The layer, for a subset of tokens.                                   */
/* out[i, h] = sum_s w[t,s] * fc2_e( act( fc1_e(x_t) ) )[h], t = tokens[i] */
/* ------------------------------------------------------------------ */
/* One projection row's dot product with x, plus its bias entry. */
static double row_dot(const uint8_t* codes, const uint16_t* scales, const uint8_t* zp,
                      int64_t row, const double* x, int32_t K, int32_t bits, int32_t block_size,
                      double zpo, int32_t dtype, const float* bias, double* wrow)
{
    dequant_row(codes, scales, zp, row, K, bits, block_size, zpo, dtype, NULL, wrow);
    double acc = 0.0;
    for (int32_t k = 0; k < K; ++k) {
        acc += x[k] * wrow[k];
    }
    return acc + (bias ? (double)bias[row] : 0.0);
}

void oracle_forward(const uint16_t* hidden, const float* logits, int64_t T, int32_t H, int32_t I,
                    int32_t E, const uint8_t* fc1_codes, const uint16_t* fc1_scales,
                    const uint8_t* fc1_zp, int32_t fc1_bits, const uint8_t* fc2_codes,
                    const uint16_t* fc2_scales, const uint8_t* fc2_zp, int32_t fc2_bits,
                    double zpo, int32_t block_size, int32_t top_k, int32_t normalize,
                    int32_t activation, int32_t dtype, const int64_t* tokens, int64_t n_tokens,
                    const oracle_opts* opts, double* out)
{
    (void)T;
    const oracle_opts none = {NULL, NULL, NULL, NULL, NULL, 0, NULL, NULL, 1, 1.0, 0.0, INFINITY};
    const oracle_opts* o = opts ? opts : &none;
    const act_params ap = {o->alpha, o->beta, o->limit};
    const int fusion = o->swiglu_fusion;
    const int64_t N1 = fusion == 0 ? (int64_t)I : 2 * (int64_t)I;  /* rows of fc1 per expert */
    const int64_t widest = H > I ? H : I;
#pragma omp parallel
    {
        ranked_expert* scratch = (ranked_expert*)malloc(sizeof(ranked_expert) * (size_t)E);
        int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)top_k);
        double* w = (double*)malloc(sizeof(double) * (size_t)top_k);
        double* x = (double*)malloc(sizeof(double) * (size_t)H);
        double* wrow = (double*)malloc(sizeof(double) * (size_t)widest);
        double* a = (double*)malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_tokens; ++i) {
            const int64_t t = tokens[i];
            double* out_row = out + i * H;
            route_one(logits + t * E, o->router_weights ? o->router_weights + t * E : NULL, E,
                      top_k, normalize, scratch, ids, w);
            for (int32_t h = 0; h < H; ++h) {
                x[h] = widen(hidden[t * H + h], dtype);
                out_row[h] = 0.0;
            }
            for (int32_t s = 0; s < top_k; ++s) {
                const int64_t e = ids[s];
                for (int32_t j = 0; j < I; ++j) {             /* fc1 (+ fc3), activation */
                    int64_t gate_row, up_row;
                    if (fusion == 1) {
                        gate_row = 2 * (int64_t)j;
                        up_row = 2 * (int64_t)j + 1;
                    } else {
                        gate_row = j;
                        up_row = fusion == 2 ? (int64_t)I + j : j;
                    }
                    const double g = row_dot(fc1_codes, fc1_scales, fc1_zp, e * N1 + gate_row, x, H,
                                             fc1_bits, block_size, zpo, dtype, o->fc1_bias, wrow);
                    const double u =
                        fusion == 0
                            ? row_dot(o->fc3_codes, o->fc3_scales, o->fc3_zp, e * (int64_t)I + up_row,
                                      x, H, o->fc3_bits, block_size, zpo, dtype, o->fc3_bias, wrow)
                            : row_dot(fc1_codes, fc1_scales, fc1_zp, e * N1 + up_row, x, H, fc1_bits,
                                      block_size, zpo, dtype, o->fc1_bias, wrow);
                    a[j] = gated(g, u, activation, &ap);
                }
                for (int32_t h = 0; h < H; ++h) {             /* fc2, then weighted sum */
                    const double y = row_dot(fc2_codes, fc2_scales, fc2_zp, e * (int64_t)H + h, a, I,
                                             fc2_bits, block_size, zpo, dtype, o->fc2_bias, wrow);
                    out_row[h] += w[s] * y;
                }
            }
        }
        free(scratch);
        free(ids);
        free(w);
        free(x);
        free(wrow);
        free(a);
    }
}

/* ------------------------------------------------------------------ */
/* Shared expert  [moe.rs: a shared gate GEMM gives one logit per token,   */
/* a shared gate/up GEMM, the gated activation and a shared down GEMM     */
/* give the shared output, and the token-gated add puts the sigmoid of    */
/* the token's logit times that output onto the routed output].          */
/* Here the shared projections have the experts' packed format (one       */
/* expert, fc1 rows gate/up interleaved) and the shared gate is a dtype   */
/* vector g[H]:                                                           */
/*   out[i, h] = sigmoid(sum_h' x[t,h'] g[h']) * fc2_s(act(fc1_s(x_t)))[h] */
/* with t = tokens[i]; the caller adds it to the routed layer output.     */
/* ------------------------------------------------------------------ */
static double sigmoid(double z)
{
    return 1.0 / (1.0 + exp(-z));
}

void oracle_shared_expert(const uint16_t* hidden, int64_t T, int32_t H, int32_t Is,
                          const uint8_t* fc1_codes, const uint16_t* fc1_scales,
                          const uint8_t* fc1_zp, int32_t fc1_bits, const uint8_t* fc2_codes,
                          const uint16_t* fc2_scales, const uint8_t* fc2_zp, int32_t fc2_bits,
                          double zpo, int32_t block_size, int32_t activation, int32_t dtype,
                          const uint16_t* gate, const int64_t* tokens, int64_t n_tokens,
                          double* out)
{
    (void)T;
    const int64_t N1 = 2 * (int64_t)Is;
    const int64_t widest = H > Is ? H : Is;
#pragma omp parallel
    {
        double* x = (double*)malloc(sizeof(double) * (size_t)H);
        double* wrow = (double*)malloc(sizeof(double) * (size_t)widest);
        double* y1 = (double*)malloc(sizeof(double) * (size_t)N1);
        double* a = (double*)malloc(sizeof(double) * (size_t)Is);
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_tokens; ++i) {
            const int64_t t = tokens[i];
            double logit = 0.0;
            for (int32_t h = 0; h < H; ++h) {
                x[h] = widen(hidden[t * H + h], dtype);
                logit += x[h] * widen(gate[h], dtype);
            }
            const double g = sigmoid(logit);
            for (int64_t n = 0; n < N1; ++n) {                  /* shared gate/up */
                dequant_row(fc1_codes, fc1_scales, fc1_zp, n, H, fc1_bits, block_size, zpo, dtype,
                            NULL, wrow);
                double acc = 0.0;
                for (int32_t h = 0; h < H; ++h) {
                    acc += x[h] * wrow[h];
                }
                y1[n] = acc;
            }
            const act_params plain = {1.0, 0.0, INFINITY};
            for (int32_t j = 0; j < Is; ++j) {
                a[j] = gated(y1[2 * j], y1[2 * j + 1], activation, &plain);
            }
            for (int32_t h = 0; h < H; ++h) {                   /* shared down, gated */
                dequant_row(fc2_codes, fc2_scales, fc2_zp, h, Is, fc2_bits, block_size, zpo, dtype,
                            NULL, wrow);
                double acc = 0.0;
                for (int32_t j = 0; j < Is; ++j) {
                    acc += a[j] * wrow[j];
                }
                out[i * H + h] = g * acc;
            }
        }
        free(x);
        free(wrow);
        free(y1);
        free(a);
    }
}

/* ------------------------------------------------------------------ */
/* Expert grouping and tile work-list                                   */
/* [qmoe.rs, launch_grouping: counts, offsets, grouped routes];         */
/* [gemm_quant_moe.rs, moe_build_tile_worklist: experts ascending]      */
/* Route ids with an expert outside [0, E) are left out of every group. */
/* ------------------------------------------------------------------ */
void oracle_group(const int32_t* ids, int64_t R, int32_t E, int32_t m_tile, int32_t n_tile,
                  int32_t N, int32_t* offsets, int32_t* sorted_routes, int32_t* worklist,
                  int64_t capacity, int64_t* n_items)
{
    int64_t* cursor = (int64_t*)calloc((size_t)E + 1, sizeof(int64_t));
    for (int64_t r = 0; r < R; ++r) {
        if (ids[r] >= 0 && ids[r] < E) {
            cursor[ids[r] + 1] += 1;
        }
    }
    for (int32_t e = 0; e < E; ++e) {                      /* exclusive scan */
        cursor[e + 1] += cursor[e];
    }
    for (int32_t e = 0; e <= E; ++e) {
        offsets[e] = (int32_t)cursor[e];
    }
    for (int64_t r = 0; r < R; ++r) {                      /* stable placement */
        if (ids[r] >= 0 && ids[r] < E) {
            sorted_routes[cursor[ids[r]]++] = (int32_t)r;
        }
    }
    const int64_t n_tiles = ((int64_t)N + n_tile - 1) / n_tile;
    int64_t w = 0;
    for (int32_t e = 0; e < E; ++e) {
        const int64_t rows = offsets[e + 1] - offsets[e];
        const int64_t m_tiles = (rows + m_tile - 1) / m_tile;
        for (int64_t m = 0; m < m_tiles; ++m) {
            for (int64_t n = 0; n < n_tiles; ++n, ++w) {
                if (w < capacity) {
                    worklist[3 * w + 0] = e;
                    worklist[3 * w + 1] = (int32_t)m;
                    worklist[3 * w + 2] = (int32_t)n;
                }
            }
        }
    }
    *n_items = w;
    free(cursor);
}
