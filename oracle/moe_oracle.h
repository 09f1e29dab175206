/*
 * CPU oracle for the MoE layer forward -- TEST INFRASTRUCTURE ONLY.
 *
 * This is the plain, slow, obviously-correct statement of what the layer
 * computes, used to check the GPU library. Only the tests, the smoke entry
 * and the benchmark's CPU-baseline leg may load it. It shares no source with
 * the GPU library (its own bf16, e2m1 and e8m0 decoders, its own rounding).
 *
 * Precision: the router is fp32 (the pages fix it); everything after the
 * router is computed in double and rounded once where the layer's contract
 * says a value is stored in a narrower type (H and y in bf16; x and H in
 * MXFP8 for OR_MXFP4_A8 weights).
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* OR_MXFP4_A8: MXFP4 weights whose products take the activation operands
 * (the x rows and H of the routed experts) as MXFP8 e4m3 blocks. */
enum { OR_F32 = 0, OR_BF16 = 1, OR_MXFP4 = 2, OR_MXFP4_A8 = 3 };
enum { OR_SOFTMAX = 0, OR_SIGMOID = 1, OR_SQRT_SOFTPLUS = 2 };

typedef struct {
  int32_t T, D, E, F, k;
  int32_t gating;     /* OR_SOFTMAX / OR_SIGMOID / OR_SQRT_SOFTPLUS */
  int32_t renorm;     /* 1: divide the k weights by their sum */
  int32_t capacity;   /* <= 0: unlimited */
  float clamp;        /* <= 0: none; else gate and up clamped to [-clamp, clamp] */
  int32_t act;        /* OR_F32 or OR_BF16 */
  int32_t wdt;        /* OR_F32, OR_BF16, OR_MXFP4 or OR_MXFP4_A8 */
  int32_t shared_F;   /* 0: no shared expert */
} oracle_cfg;

typedef struct {
  const void *W_gate, *W_up, *W_down;      /* codes for MXFP4 */
  const uint8_t *S_gate, *S_up, *S_down;   /* e8m0 scales for MXFP4 */
  const uint16_t *Ws_gate, *Ws_up, *Ws_down; /* shared expert, bf16 */
} oracle_weights;

double oracle_bf16_to_double(uint16_t b);
uint16_t oracle_double_to_bf16(double v);
void oracle_double_to_bf16_array(const double* v, int64_t n, uint16_t* out);
double oracle_e2m1(unsigned code);
double oracle_e8m0(unsigned s);
double oracle_e4m3(unsigned code);
unsigned oracle_e4m3_encode(double v);
void oracle_mxfp8_quantize(const double* v, int n, uint8_t* codes, uint8_t* scales);
double oracle_softplus(double s);
double oracle_silu(double z);
int oracle_capacity_formula(int S, int top_k, int num_experts);

void oracle_router_logits(const oracle_cfg* c, const void* x, const float* W_r, float* logits);
void oracle_select_topk(const oracle_cfg* c, const float* logits, const float* bias, int32_t* topk_idx);
void oracle_gate_weights(const oracle_cfg* c, const float* logits, const float* bias,
                         const int32_t* topk_idx, float* topk_w);
void oracle_dispatch(const oracle_cfg* c, const int32_t* topk_idx, int32_t* counts,
                     int32_t* offsets, int32_t* slot_pos, int32_t* perm_token);
void oracle_expert_rows(const oracle_cfg* c, const oracle_weights* w, int expert, int nrows,
                        const void* x, const int32_t* rows, double* h_out, double* o_out);
void oracle_shared_rows(const oracle_cfg* c, const oracle_weights* w, int nrows,
                        const void* x, const int32_t* rows, double* o_out);
void oracle_forward_tokens(const oracle_cfg* c, const oracle_weights* w, const void* x,
                           const int32_t* topk_idx, const float* topk_w, const int32_t* slot_pos,
                           int ntok, const int32_t* tokens, double* y_exact, void* y_out);

#ifdef __cplusplus
}
#endif
#endif
