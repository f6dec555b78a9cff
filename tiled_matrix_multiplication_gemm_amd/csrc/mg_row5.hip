// Kernels of table row 5 (see mg_table.h).
#include "mg_launch.h"

MG_DEFINE_ROW(5, Cfg5, void)
MG_DEFINE_ROW_TAIL(5, void)
