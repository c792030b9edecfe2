// Single device translation unit of librax: every kernel and the device error word
// live in one code object (no relocatable device code needed).
#include "kv_scatter.hip"
#include "attention.hip"
#include "projection.hip"
