// Kernels of table row 7 (see mg_table.h).
#include "mg_launch.h"

MG_DEFINE_ROW(7, Cfg7, Fast7)
MG_DEFINE_ROW_TAIL(7, Fast7)
