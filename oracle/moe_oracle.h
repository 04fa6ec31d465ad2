/* Plain fp64 CPU oracle for the routed-expert MoE FFN layer.
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg; never by the GPU library.
 * All pointers are host pointers in the canonical layout (see moe_oracle.c). */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

typedef struct {
  int d, E, K, f, fs;
  const int8_t* router_w;        /* [E][d] */
  const uint16_t* router_scale;  /* [E] fp16 */
  const float* router_bias;      /* [E] or NULL */
  const uint32_t *gate_q, *up_q, *down_q;          /* [E][f][d/8], [E][f][d/8], [E][d][f/8] */
  const uint16_t *gate_s, *gate_b, *up_s, *up_b;   /* [E][f][d/64] fp16 */
  const uint16_t *down_s, *down_b;                 /* [E][d][f/64] fp16 */
  const uint32_t *sh_gate_q, *sh_up_q, *sh_down_q; /* [fs][d/8], [fs][d/8], [d][fs/8] */
  const uint16_t *sh_gate_s, *sh_gate_b, *sh_up_s, *sh_up_b, *sh_down_s, *sh_down_b;
} oracle_layer;

int oracle_threads(void);
void oracle_set_threads(int n);
double oracle_f16_to_f64(uint16_t h);
double oracle_bf16_to_f64(uint16_t b);
uint16_t oracle_f64_to_bf16(double v);
double oracle_weight(const uint32_t* q, const uint16_t* s, const uint16_t* b, int cols, int r, int c);
void oracle_dequant(const uint32_t* q, const uint16_t* s, const uint16_t* b, int rows, int cols, double* W);
void oracle_router_logits(const oracle_layer* L, const double* x, int T, double* logits);
void oracle_select_one(const double* l, int E, int K, int32_t* ids, double* w, double* margin);
void oracle_weights_for_set(const double* l, const int32_t* sel, int K, double* w);
void oracle_expert(const oracle_layer* L, int expert, const double* x, double* out);
int oracle_layer_forward(const oracle_layer* L, const double* x, int T, const int32_t* forced, double* y,
                         int32_t* ids_out, double* w_out, double* margin_out);
void oracle_sort(const int32_t* ids, int T, int K, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
                 int32_t* inv);
void oracle_rmsnorm_bf16(const uint16_t* h, int d, double eps, uint16_t* n_out);
void oracle_residual_bf16(const uint16_t* h, const double* y, int d, uint16_t* h_out);
int oracle_stack_step(const oracle_layer* layers, int n_layers, double eps, uint16_t* h, const int32_t* forced,
                      int32_t* ids_out);
#endif
