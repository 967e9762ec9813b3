// libmoe.hip — single translation unit of libmoe (one device error word,
// one code object).  Each included file holds one stage of the path.
#include "ffn_decode.hip"
#include "quant.hip"
#include "route.hip"
#include "router.hip"
#include "ffn_mfma.hip"
#include "ffn_int8.hip"
#include "decode_fused.hip"
#include "moe_api.hip"
